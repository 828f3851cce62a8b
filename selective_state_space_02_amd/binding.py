"""Thin ctypes binding of libssmscan.so (argument marshalling only).

Each function has the name of the C entry point it calls and takes torch tensors that
live on the GPU.  It checks what the C ABI cannot see (device, dtype, contiguity --
a strided view read as dense silently gives wrong numbers), allocates missing outputs
and the workspace with torch, and calls the library on torch's current stream.  All
arithmetic runs in the library's HIP kernels; nothing here computes any part of the
scan, the conv or the norm.  If the library is missing or cannot be loaded, every call
raises RuntimeError: there is no fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssmscan.so")

SSM_F32, SSM_BF16 = 0, 1
SSM_OK, SSM_ERR_ARG, SSM_ERR_UNSUPPORTED, SSM_ERR_WORKSPACE, SSM_ERR_ALIGN, SSM_ERR_HIP = (
    0, -1, -2, -3, -4, -5)

EXPORTS = ("ssm_last_error", "ssm_version", "ssm_set_kernel_timer", "ssm_scan_ckpt_bytes",
           "ssm_scan_fwd_workspace_bytes", "ssm_scan_bwd_workspace_bytes", "ssm_scan_fwd",
           "ssm_scan_bwd", "conv1d_causal_bwd_workspace_bytes", "conv1d_causal_bwd",
           "rmsnorm_bwd_workspace_bytes", "rmsnorm_bwd", "conv1d_causal_fwd", "rmsnorm_fwd",
           "ssm_scan_step", "conv1d_causal_step", "ssm_scan_fused_fwd", "ssm_scan_fused_bwd",
           "ssm_scan_fused_step", "ssm_decode_step", "ssm_scan_chunks",
           "ssm_scan_ckpt_bytes_every", "ssm_scan_bwd_workspace_bytes_every",
           "ssm_scan_fwd_every", "ssm_scan_bwd_every", "rmsnorm_bwd_noalloc",
           "ssm_alpha_scan_bwd_workspace_bytes", "ssm_alpha_scan_fwd", "ssm_alpha_scan_bwd")

_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int64
_S = ctypes.c_size_t
_E = ctypes.c_int


class SsmError(RuntimeError):
    """A non-OK status from the library (code in .code)."""

    def __init__(self, code, msg):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def load():
    """Load libssmscan.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                           "(build it with: python selective_state_space_02_amd/build.py)")
    try:
        lib = ctypes.CDLL(LIB_PATH)
    except OSError as e:
        raise RuntimeError(f"cannot load {LIB_PATH}: {e}") from e
    lib.ssm_last_error.restype = ctypes.c_char_p
    lib.ssm_last_error.argtypes = []
    lib.ssm_version.restype = ctypes.c_char_p
    lib.ssm_version.argtypes = []
    lib.ssm_set_kernel_timer.restype = _E
    lib.ssm_set_kernel_timer.argtypes = [_E, _P, _P]
    lib.ssm_scan_ckpt_bytes.restype = _S
    lib.ssm_scan_ckpt_bytes.argtypes = [_I] * 4
    lib.ssm_scan_chunks.restype = _E
    lib.ssm_scan_chunks.argtypes = [_I] * 4 + [ctypes.POINTER(ctypes.c_int)] * 2
    lib.ssm_scan_fwd_workspace_bytes.restype = _S
    lib.ssm_scan_fwd_workspace_bytes.argtypes = [_I] * 4 + [_E]
    lib.ssm_scan_bwd_workspace_bytes.restype = _S
    lib.ssm_scan_bwd_workspace_bytes.argtypes = [_I] * 4 + [_E, _E]
    lib.ssm_scan_fwd.restype = _E
    lib.ssm_scan_fwd.argtypes = [_P, _E] + [_I] * 4 + [_P] * 10 + [_P, _S]
    lib.ssm_scan_bwd.restype = _E
    lib.ssm_scan_bwd.argtypes = [_P, _E] + [_I] * 4 + [_P] * 16 + [_P, _S]
    lib.ssm_scan_ckpt_bytes_every.restype = _S
    lib.ssm_scan_ckpt_bytes_every.argtypes = [_I] * 5
    lib.ssm_scan_bwd_workspace_bytes_every.restype = _S
    lib.ssm_scan_bwd_workspace_bytes_every.argtypes = [_I] * 4 + [_E, _E, _I, _I]
    lib.ssm_scan_fwd_every.restype = _E
    lib.ssm_scan_fwd_every.argtypes = [_P, _E] + [_I] * 4 + [_P] * 10 + [_I] + [_P, _S]
    lib.ssm_scan_bwd_every.restype = _E
    lib.ssm_scan_bwd_every.argtypes = [_P, _E] + [_I] * 4 + [_P] * 17 + [_I, _I] + [_P, _S]
    lib.ssm_scan_fused_fwd.restype = _E
    lib.ssm_scan_fused_fwd.argtypes = [_P, _E] + [_I] * 4 + [_P] * 8 + [_E] + [_P] * 5 + [_P, _S]
    lib.ssm_scan_fused_bwd.restype = _E
    lib.ssm_scan_fused_bwd.argtypes = [_P, _E] + [_I] * 4 + [_P] * 8 + [_E] + [_P] * 13 + [_P, _S]
    lib.conv1d_causal_bwd_workspace_bytes.restype = _S
    lib.conv1d_causal_bwd_workspace_bytes.argtypes = [_I] * 4 + [_E]
    lib.conv1d_causal_bwd.restype = _E
    lib.conv1d_causal_bwd.argtypes = [_P, _E] + [_I] * 4 + [_P] * 3 + [_E] + [_P] * 4 + [_P, _S]
    lib.rmsnorm_bwd_workspace_bytes.restype = _S
    lib.rmsnorm_bwd_workspace_bytes.argtypes = [_I] * 2 + [_E]
    lib.rmsnorm_bwd.restype = _E
    lib.rmsnorm_bwd.argtypes = [_P, _E] + [_I] * 2 + [_P] * 6 + [_P, _S]
    lib.rmsnorm_bwd_noalloc.restype = _E
    lib.rmsnorm_bwd_noalloc.argtypes = [_P, _E] + [_I] * 2 + [_P] * 6
    lib.ssm_alpha_scan_bwd_workspace_bytes.restype = _S
    lib.ssm_alpha_scan_bwd_workspace_bytes.argtypes = [_I] * 4
    lib.ssm_alpha_scan_fwd.restype = _E
    lib.ssm_alpha_scan_fwd.argtypes = [_P] + [_I] * 4 + [_P] * 5
    lib.ssm_alpha_scan_bwd.restype = _E
    lib.ssm_alpha_scan_bwd.argtypes = [_P] + [_I] * 4 + [_P] * 8 + [_P, _S]
    lib.conv1d_causal_fwd.restype = _E
    lib.conv1d_causal_fwd.argtypes = [_P, _E] + [_I] * 4 + [_P] * 3 + [_E, _P]
    lib.rmsnorm_fwd.restype = _E
    lib.rmsnorm_fwd.argtypes = [_P, _E] + [_I] * 2 + [_P, _P, _P, ctypes.c_float, _P, _P, _P]
    lib.ssm_scan_step.restype = _E
    lib.ssm_scan_step.argtypes = [_P, _E] + [_I] * 3 + [_P] * 8
    lib.conv1d_causal_step.restype = _E
    lib.conv1d_causal_step.argtypes = [_P, _E] + [_I] * 3 + [_P] * 4 + [_E, _P]
    lib.ssm_scan_fused_step.restype = _E
    lib.ssm_decode_step.restype = _E
    lib.ssm_decode_step.argtypes = [_P, _E] + [_I] * 4 + [_P] * 11 + [_E, _P, _P]
    lib.ssm_scan_fused_step.argtypes = [_P, _E] + [_I] * 3 + [_P] * 8 + [_E, _P, _P]
    _lib = lib
    return lib


def last_error() -> str:
    return load().ssm_last_error().decode()


def version() -> str:
    return load().ssm_version().decode()


KERNEL_IDS = {"fwd_summary": 1, "fwd_carry": 2, "fwd_output": 3, "bwd_summary": 4,
              "bwd_carry": 5, "bwd_main": 6, "conv_bwd": 7, "rms_bwd": 8, "conv_fwd": 9,
              "rms_fwd": 10, "scan_step": 11, "conv_step": 12, "decode_step": 13,
              "ckpt_regen": 14}


def ssm_set_kernel_timer(kernel, start=None, stop=None):
    """Arm (a pair of raw hipEvent_t handles, as ints) or disarm (None, None) the timing
    hook around one kernel, named as in KERNEL_IDS or by its id."""
    kid = KERNEL_IDS.get(kernel, kernel)
    sp = ctypes.c_void_p(start) if start is not None else None
    ep = ctypes.c_void_p(stop) if stop is not None else None
    _check(load().ssm_set_kernel_timer(int(kid), sp, ep))


def _check(rc):
    if rc != SSM_OK:
        raise SsmError(rc, last_error())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SSM_F32
    if t.dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError(f"activation dtype must be float32 or bfloat16, got {t.dtype}")


def _ptr(t, name, dtype=None, shape=None, device=None):
    """Device pointer of a dense tensor (None -> NULL), after the checks the ABI needs."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor (got device {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous (strided views are not accepted)")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes, device, ws):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace too small: {ws.numel() * ws.element_size()} < {nbytes} bytes")
    return ws, ws.numel() * ws.element_size()


# ----------------------------------------------------------------------------------
# selective scan
# ----------------------------------------------------------------------------------

def ssm_scan_ckpt_bytes(B, L, D, N) -> int:
    return int(load().ssm_scan_ckpt_bytes(B, L, D, N))


def ssm_scan_ckpt_bytes_every(B, L, D, N, ck_every) -> int:
    return int(load().ssm_scan_ckpt_bytes_every(B, L, D, N, ck_every))


def ssm_scan_bwd_workspace_bytes_every(B, L, D, N, dtype_code, with_ckpt, ck_every, slabs) -> int:
    return int(load().ssm_scan_bwd_workspace_bytes_every(B, L, D, N, dtype_code,
                                                         int(bool(with_ckpt)), ck_every, slabs))


def ssm_scan_fwd_workspace_bytes(B, L, D, N, dtype_code) -> int:
    return int(load().ssm_scan_fwd_workspace_bytes(B, L, D, N, dtype_code))


def ssm_scan_bwd_workspace_bytes(B, L, D, N, dtype_code, with_ckpt) -> int:
    return int(load().ssm_scan_bwd_workspace_bytes(B, L, D, N, dtype_code, int(bool(with_ckpt))))


def new_ckpt(B, L, D, N, device, ck_every=0) -> torch.Tensor:
    """A buffer for the forward's checkpoints (f32, opaque layout) at the given interval
    (0: the default)."""
    nbytes = ssm_scan_ckpt_bytes_every(B, L, D, N, ck_every)
    if nbytes == 0:
        raise ValueError(f"unsupported checkpoint interval {ck_every}")
    return torch.empty(nbytes // 4, dtype=torch.float32, device=device)


def ssm_scan_fwd(x, delta, A, Bm, Cm, Dv, h0=None, y=None, ckpt=None, h_last=None, ws=None):
    """y = scan(x, delta, A, Bm, Cm, Dv; h0).  Returns y (allocated if not given)."""
    return ssm_scan_fwd_every(x, delta, A, Bm, Cm, Dv, 0, h0=h0, y=y, ckpt=ckpt, h_last=h_last,
                              ws=ws)


def ssm_scan_fwd_every(x, delta, A, Bm, Cm, Dv, ck_every, h0=None, y=None, ckpt=None,
                       h_last=None, ws=None):
    """ssm_scan_fwd saving its states every ck_every steps (0: the default interval, which
    calls ssm_scan_fwd itself)."""
    lib = load()
    Bsz, L, D = x.shape
    N = A.shape[1]
    dev = x.device
    dt = x.dtype
    code = _dtype_code(x)
    if y is None:
        y = torch.empty_like(x)
    args = [
        _ptr(x, "x", dt, (Bsz, L, D), dev), _ptr(delta, "delta", dt, (Bsz, L, D), dev),
        _ptr(A, "A", torch.float32, (D, N), dev), _ptr(Bm, "Bm", dt, (Bsz, L, N), dev),
        _ptr(Cm, "Cm", dt, (Bsz, L, N), dev), _ptr(Dv, "Dv", torch.float32, (D,), dev),
        _ptr(h0, "h0", torch.float32, (Bsz, D, N), dev), _ptr(y, "y", dt, (Bsz, L, D), dev),
        _ptr(ckpt, "ckpt", torch.float32, None, dev),
        _ptr(h_last, "h_last", torch.float32, (Bsz, D, N), dev),
    ]
    if ckpt is not None and ckpt.numel() * 4 < ssm_scan_ckpt_bytes_every(Bsz, L, D, N, ck_every):
        raise ValueError("ckpt buffer too small (use new_ckpt)")
    need = ssm_scan_fwd_workspace_bytes(Bsz, L, D, N, code)
    ws, nbytes = _workspace(need, dev, ws)
    wsp = _ptr(ws, "ws") if ws is not None else None
    if ck_every == 0:
        _check(lib.ssm_scan_fwd(_stream(dev), code, Bsz, L, D, N, *args, wsp, nbytes))
    else:
        _check(lib.ssm_scan_fwd_every(_stream(dev), code, Bsz, L, D, N, *args, ck_every, wsp,
                                      nbytes))
    return y


def ssm_scan_bwd(x, delta, A, Bm, Cm, Dv, dy, ckpt=None, h0=None, dx=None, ddelta=None,
                 dA=None, dB=None, dC=None, dD=None, dh0=None, ws=None):
    """Backward.  dA and dD are accumulated into (zeros allocated if not given); every
    other gradient is overwritten.  Returns dict dx, ddelta, dA, dB, dC, dD, dh0."""
    return ssm_scan_bwd_every(x, delta, A, Bm, Cm, Dv, dy, 0, 1, ckpt=ckpt, h0=h0, dx=dx,
                              ddelta=ddelta, dA=dA, dB=dB, dC=dC, dD=dD, dh0=dh0, ws=ws)


def ssm_scan_bwd_every(x, delta, A, Bm, Cm, Dv, dy, ck_every, slabs, ckpt=None, h0=None, dx=None,
                       ddelta=None, dA=None, dB=None, dC=None, dD=None, dh0=None, dh_last=None,
                       ws=None):
    """ssm_scan_bwd from checkpoints saved every ck_every steps, regenerating the dense
    states slab by slab (ck_every = 0 and slabs = 1 call ssm_scan_bwd itself, unless
    dh_last, the gradient arriving at the final state [B, D, N] f32, is given)."""
    lib = load()
    Bsz, L, D = x.shape
    N = A.shape[1]
    dev = x.device
    dt = x.dtype
    code = _dtype_code(x)
    f32 = torch.float32
    dx = torch.empty_like(x) if dx is None else dx
    ddelta = torch.empty_like(x) if ddelta is None else ddelta
    dA = torch.zeros((D, N), dtype=f32, device=dev) if dA is None else dA
    dB = torch.empty((Bsz, L, N), dtype=f32, device=dev) if dB is None else dB
    dC = torch.empty((Bsz, L, N), dtype=f32, device=dev) if dC is None else dC
    dD = torch.zeros((D,), dtype=f32, device=dev) if dD is None else dD
    if ckpt is not None and ckpt.numel() * 4 < ssm_scan_ckpt_bytes_every(Bsz, L, D, N, ck_every):
        raise ValueError("ckpt buffer too small")
    args = [
        _ptr(x, "x", dt, (Bsz, L, D), dev), _ptr(delta, "delta", dt, (Bsz, L, D), dev),
        _ptr(A, "A", f32, (D, N), dev), _ptr(Bm, "Bm", dt, (Bsz, L, N), dev),
        _ptr(Cm, "Cm", dt, (Bsz, L, N), dev), _ptr(Dv, "Dv", f32, (D,), dev),
        _ptr(h0, "h0", f32, (Bsz, D, N), dev), _ptr(dy, "dy", dt, (Bsz, L, D), dev),
        _ptr(ckpt, "ckpt", f32, None, dev),
        _ptr(dx, "dx", dt, (Bsz, L, D), dev), _ptr(ddelta, "ddelta", dt, (Bsz, L, D), dev),
        _ptr(dA, "dA", f32, (D, N), dev), _ptr(dB, "dB", f32, (Bsz, L, N), dev),
        _ptr(dC, "dC", f32, (Bsz, L, N), dev), _ptr(dD, "dD", f32, (D,), dev),
        _ptr(dh0, "dh0", f32, (Bsz, D, N), dev),
    ]
    dhl = _ptr(dh_last, "dh_last", f32, (Bsz, D, N), dev)
    if ssm_scan_ckpt_bytes_every(Bsz, L, D, N, ck_every) == 0 or not 1 <= slabs <= 65536:
        raise ValueError(f"unsupported checkpoint interval {ck_every} or slabs {slabs}")
    need = ssm_scan_bwd_workspace_bytes_every(Bsz, L, D, N, code, ckpt is not None, ck_every,
                                              slabs)
    ws, nbytes = _workspace(need, dev, ws)
    wsp = _ptr(ws, "ws") if ws is not None else None
    if ck_every == 0 and slabs == 1 and dh_last is None:
        _check(lib.ssm_scan_bwd(_stream(dev), code, Bsz, L, D, N, *args, wsp, nbytes))
    else:
        _check(lib.ssm_scan_bwd_every(_stream(dev), code, Bsz, L, D, N, *args, dhl, ck_every,
                                      slabs, wsp, nbytes))
    return dict(dx=dx, ddelta=ddelta, dA=dA, dB=dB, dC=dC, dD=dD, dh0=dh0)


def ssm_scan_fused_fwd(x, delta, A, Bm, Cm, Dv, h0=None, delta_bias=None, delta_softplus=False,
                       z=None, out=None, y_save=None, ckpt=None, h_last=None, ws=None):
    """The scan with its Mamba-block neighbours: time step softplus(delta + delta_bias)
    (or delta + delta_bias), output y * silu(z) when z is given.  y_save (with z) receives
    y before the gate, which the backward needs.  Returns out."""
    lib = load()
    Bsz, L, D = x.shape
    N = A.shape[1]
    dev = x.device
    dt = x.dtype
    code = _dtype_code(x)
    f32 = torch.float32
    out = torch.empty_like(x) if out is None else out
    if ckpt is not None and ckpt.numel() * 4 < ssm_scan_ckpt_bytes(Bsz, L, D, N):
        raise ValueError("ckpt buffer too small (use new_ckpt)")
    args = [
        _ptr(x, "x", dt, (Bsz, L, D), dev), _ptr(delta, "delta", dt, (Bsz, L, D), dev),
        _ptr(A, "A", f32, (D, N), dev), _ptr(Bm, "Bm", dt, (Bsz, L, N), dev),
        _ptr(Cm, "Cm", dt, (Bsz, L, N), dev), _ptr(Dv, "Dv", f32, (D,), dev),
        _ptr(h0, "h0", f32, (Bsz, D, N), dev), _ptr(delta_bias, "delta_bias", f32, (D,), dev),
        1 if delta_softplus else 0, _ptr(z, "z", dt, (Bsz, L, D), dev),
        _ptr(out, "out", dt, (Bsz, L, D), dev), _ptr(y_save, "y_save", dt, (Bsz, L, D), dev),
        _ptr(ckpt, "ckpt", f32, None, dev), _ptr(h_last, "h_last", f32, (Bsz, D, N), dev),
    ]
    need = ssm_scan_fwd_workspace_bytes(Bsz, L, D, N, code)
    ws, nbytes = _workspace(need, dev, ws)
    _check(lib.ssm_scan_fused_fwd(_stream(dev), code, Bsz, L, D, N, *args,
                                  _ptr(ws, "ws") if ws is not None else None, nbytes))
    return out


def ssm_scan_fused_bwd(x, delta, A, Bm, Cm, Dv, dout, ckpt=None, h0=None, delta_bias=None,
                       delta_softplus=False, z=None, y_save=None, dx=None, ddelta=None,
                       dA=None, dB=None, dC=None, dD=None, dh0=None, dz=None,
                       ddelta_bias=None, ws=None):
    """Backward of ssm_scan_fused_fwd for upstream dout of its output.  dA, dD and
    ddelta_bias are accumulated into (zeros allocated if not given; ddelta_bias only when
    delta_bias is given); every other gradient is overwritten.  With z, y_save is
    required.  Returns dict dx, ddelta, dA, dB, dC, dD, dh0, dz, ddelta_bias."""
    lib = load()
    Bsz, L, D = x.shape
    N = A.shape[1]
    dev = x.device
    dt = x.dtype
    code = _dtype_code(x)
    f32 = torch.float32
    dx = torch.empty_like(x) if dx is None else dx
    ddelta = torch.empty_like(x) if ddelta is None else ddelta
    dA = torch.zeros((D, N), dtype=f32, device=dev) if dA is None else dA
    dB = torch.empty((Bsz, L, N), dtype=f32, device=dev) if dB is None else dB
    dC = torch.empty((Bsz, L, N), dtype=f32, device=dev) if dC is None else dC
    dD = torch.zeros((D,), dtype=f32, device=dev) if dD is None else dD
    if z is not None and dz is None:
        dz = torch.empty_like(x)
    if delta_bias is not None and ddelta_bias is None:
        ddelta_bias = torch.zeros((D,), dtype=f32, device=dev)
    if ckpt is not None and ckpt.numel() * 4 < ssm_scan_ckpt_bytes(Bsz, L, D, N):
        raise ValueError("ckpt buffer too small")
    args = [
        _ptr(x, "x", dt, (Bsz, L, D), dev), _ptr(delta, "delta", dt, (Bsz, L, D), dev),
        _ptr(A, "A", f32, (D, N), dev), _ptr(Bm, "Bm", dt, (Bsz, L, N), dev),
        _ptr(Cm, "Cm", dt, (Bsz, L, N), dev), _ptr(Dv, "Dv", f32, (D,), dev),
        _ptr(h0, "h0", f32, (Bsz, D, N), dev), _ptr(delta_bias, "delta_bias", f32, (D,), dev),
        1 if delta_softplus else 0, _ptr(z, "z", dt, (Bsz, L, D), dev),
        _ptr(y_save, "y_save", dt, (Bsz, L, D), dev), _ptr(dout, "dout", dt, (Bsz, L, D), dev),
        _ptr(ckpt, "ckpt", f32, None, dev),
        _ptr(dx, "dx", dt, (Bsz, L, D), dev), _ptr(ddelta, "ddelta", dt, (Bsz, L, D), dev),
        _ptr(dA, "dA", f32, (D, N), dev), _ptr(dB, "dB", f32, (Bsz, L, N), dev),
        _ptr(dC, "dC", f32, (Bsz, L, N), dev), _ptr(dD, "dD", f32, (D,), dev),
        _ptr(dh0, "dh0", f32, (Bsz, D, N), dev), _ptr(dz, "dz", dt, (Bsz, L, D), dev),
        _ptr(ddelta_bias, "ddelta_bias", f32, (D,), dev),
    ]
    need = ssm_scan_bwd_workspace_bytes(Bsz, L, D, N, code, ckpt is not None)
    ws, nbytes = _workspace(need, dev, ws)
    _check(lib.ssm_scan_fused_bwd(_stream(dev), code, Bsz, L, D, N, *args,
                                  _ptr(ws, "ws") if ws is not None else None, nbytes))
    return dict(dx=dx, ddelta=ddelta, dA=dA, dB=dB, dC=dC, dD=dD, dh0=dh0, dz=dz,
                ddelta_bias=ddelta_bias)


# ----------------------------------------------------------------------------------
# conv1d / RMSNorm
# ----------------------------------------------------------------------------------

def scan_chunks(B, L, D, N):
    """(forward chunks, backward chunks) the library splits a sequence of these sizes
    into (ssm_scan_chunks; a host-side plan query)."""
    f, b = ctypes.c_int(0), ctypes.c_int(0)
    _check(load().ssm_scan_chunks(B, L, D, N, ctypes.byref(f), ctypes.byref(b)))
    return f.value, b.value


def conv1d_causal_bwd_workspace_bytes(B, L, D, K, dtype_code) -> int:
    return int(load().conv1d_causal_bwd_workspace_bytes(B, L, D, K, dtype_code))


# activation after the conv (the C enum ssm_act_t)
ACTS = {"none": 0, "silu": 1}


def _act_code(act) -> int:
    if act not in ACTS:
        raise ValueError(f"activation {act!r} not supported (one of {sorted(ACTS)})")
    return ACTS[act]


def conv1d_causal_bwd(x, W, dout, bias=None, act="none", dx=None, dW=None, db=None, ws=None):
    """Returns dict dx (overwritten), dW, db (accumulated; zeros if not given).

    act="silu": dout is the gradient of silu(conv(x)); the SiLU backward runs in the
    kernel, which recomputes the conv output from x, W and bias."""
    lib = load()
    ac = _act_code(act)
    Bsz, L, D = x.shape
    K = W.shape[1]
    dev = x.device
    dt = x.dtype
    code = _dtype_code(x)
    f32 = torch.float32
    dx = torch.empty_like(x) if dx is None else dx
    dW = torch.zeros((D, K), dtype=f32, device=dev) if dW is None else dW
    db = torch.zeros((D,), dtype=f32, device=dev) if db is None else db
    bp = _ptr(bias, "bias", f32, (D,), dev) if bias is not None else None
    args = [_ptr(x, "x", dt, (Bsz, L, D), dev), _ptr(W, "W", f32, (D, K), dev), bp, ac,
            _ptr(dout, "dout", dt, (Bsz, L, D), dev), _ptr(dx, "dx", dt, (Bsz, L, D), dev),
            _ptr(dW, "dW", f32, (D, K), dev), _ptr(db, "db", f32, (D,), dev)]
    need = conv1d_causal_bwd_workspace_bytes(Bsz, L, D, K, code)
    ws, nbytes = _workspace(need, dev, ws)
    _check(lib.conv1d_causal_bwd(_stream(dev), code, Bsz, L, D, K, *args,
                                 _ptr(ws, "ws") if ws is not None else None, nbytes))
    return dict(dx=dx, dW=dW, db=db)


def rmsnorm_bwd_workspace_bytes(R, M, dtype_code) -> int:
    return int(load().rmsnorm_bwd_workspace_bytes(R, M, dtype_code))


def rmsnorm_bwd(dy, x, scale, rms, dx=None, dscale=None, ws=None):
    """Returns dict dx (overwritten), dscale (accumulated; zeros if not given)."""
    lib = load()
    R, M = x.shape
    dev = x.device
    dt = x.dtype
    code = _dtype_code(x)
    f32 = torch.float32
    dx = torch.empty_like(x) if dx is None else dx
    dscale = torch.zeros((M,), dtype=f32, device=dev) if dscale is None else dscale
    args = [_ptr(dy, "dy", dt, (R, M), dev), _ptr(x, "x", dt, (R, M), dev),
            _ptr(scale, "scale", f32, (M,), dev), _ptr(rms, "rms", f32, (R,), dev),
            _ptr(dx, "dx", dt, (R, M), dev), _ptr(dscale, "dscale", f32, (M,), dev)]
    need = rmsnorm_bwd_workspace_bytes(R, M, code)
    ws, nbytes = _workspace(need, dev, ws)
    _check(lib.rmsnorm_bwd(_stream(dev), code, R, M, *args,
                           _ptr(ws, "ws") if ws is not None else None, nbytes))
    return dict(dx=dx, dscale=dscale)


def rmsnorm_bwd_noalloc(dy, x, scale, rms, dx, dscale):
    """rmsnorm_bwd without a workspace (the library's static scratch); the caller passes
    the outputs, so nothing is allocated here either.  dx is overwritten, dscale
    accumulated.  Returns dict dx, dscale."""
    lib = load()
    R, M = x.shape
    dev = x.device
    dt = x.dtype
    code = _dtype_code(x)
    f32 = torch.float32
    args = [_ptr(dy, "dy", dt, (R, M), dev), _ptr(x, "x", dt, (R, M), dev),
            _ptr(scale, "scale", f32, (M,), dev), _ptr(rms, "rms", f32, (R,), dev),
            _ptr(dx, "dx", dt, (R, M), dev), _ptr(dscale, "dscale", f32, (M,), dev)]
    _check(lib.rmsnorm_bwd_noalloc(_stream(dev), code, R, M, *args))
    return dict(dx=dx, dscale=dscale)


def conv1d_causal_fwd(x, W, bias=None, act="none", out=None):
    """Returns out [B, L, D] (dtype of x); silu of the conv output when act="silu"."""
    lib = load()
    ac = _act_code(act)
    Bsz, L, D = x.shape
    K = W.shape[1]
    dev = x.device
    dt = x.dtype
    code = _dtype_code(x)
    f32 = torch.float32
    out = torch.empty_like(x) if out is None else out
    bp = _ptr(bias, "bias", f32, (D,), dev) if bias is not None else None
    _check(lib.conv1d_causal_fwd(_stream(dev), code, Bsz, L, D, K,
                                 _ptr(x, "x", dt, (Bsz, L, D), dev), _ptr(W, "W", f32, (D, K), dev),
                                 bp, ac, _ptr(out, "out", dt, (Bsz, L, D), dev)))
    return out


def rmsnorm_fwd(x, scale, eps, y=None, rms=None, residual=None, residual_out=None):
    """Returns (y [R, M] in the dtype of x, rms [R] f32).  With the residual stream
    (`residual`, same shape and dtype as x) the norm is applied to h = x + residual,
    which is written to residual_out (allocated if not given) and returned third:
    (y, rms, residual_out)."""
    lib = load()
    R, M = x.shape
    dev = x.device
    dt = x.dtype
    code = _dtype_code(x)
    f32 = torch.float32
    y = torch.empty_like(x) if y is None else y
    rms = torch.empty((R,), dtype=f32, device=dev) if rms is None else rms
    if residual is not None and residual_out is None:
        residual_out = torch.empty_like(x)
    _check(lib.rmsnorm_fwd(_stream(dev), code, R, M, _ptr(x, "x", dt, (R, M), dev),
                           _ptr(residual, "residual", dt, (R, M), dev),
                           _ptr(scale, "scale", f32, (M,), dev), float(eps),
                           _ptr(y, "y", dt, (R, M), dev), _ptr(rms, "rms", f32, (R,), dev),
                           _ptr(residual_out, "residual_out", dt, (R, M), dev)))
    return (y, rms) if residual is None else (y, rms, residual_out)


def ssm_scan_step(h, x_t, delta_t, A, B_t, C_t, Dv, y_t=None):
    """One token: advances h [B, D, N] (f32) in place; returns y_t [B, D]."""
    lib = load()
    Bsz, D, N = h.shape
    dev = x_t.device
    dt = x_t.dtype
    code = _dtype_code(x_t)
    f32 = torch.float32
    y_t = torch.empty_like(x_t) if y_t is None else y_t
    _check(lib.ssm_scan_step(_stream(dev), code, Bsz, D, N, _ptr(h, "h", f32, (Bsz, D, N), dev),
                             _ptr(x_t, "x_t", dt, (Bsz, D), dev),
                             _ptr(delta_t, "delta_t", dt, (Bsz, D), dev),
                             _ptr(A, "A", f32, (D, N), dev), _ptr(B_t, "B_t", dt, (Bsz, N), dev),
                             _ptr(C_t, "C_t", dt, (Bsz, N), dev), _ptr(Dv, "Dv", f32, (D,), dev),
                             _ptr(y_t, "y_t", dt, (Bsz, D), dev)))
    return y_t


def ssm_scan_fused_step(h, x_t, delta_t, A, B_t, C_t, Dv, delta_bias=None,
                        delta_softplus=False, z_t=None, out_t=None):
    """One token of the fused scan: advances h [B, D, N] (f32) in place with the time step
    softplus(delta_t + delta_bias) (or without the softplus); returns out_t [B, D], gated
    by silu(z_t) when z_t is given."""
    lib = load()
    Bsz, D, N = h.shape
    dev = x_t.device
    dt = x_t.dtype
    code = _dtype_code(x_t)
    f32 = torch.float32
    out_t = torch.empty_like(x_t) if out_t is None else out_t
    _check(lib.ssm_scan_fused_step(_stream(dev), code, Bsz, D, N,
                                   _ptr(h, "h", f32, (Bsz, D, N), dev),
                                   _ptr(x_t, "x_t", dt, (Bsz, D), dev),
                                   _ptr(delta_t, "delta_t", dt, (Bsz, D), dev),
                                   _ptr(A, "A", f32, (D, N), dev),
                                   _ptr(B_t, "B_t", dt, (Bsz, N), dev),
                                   _ptr(C_t, "C_t", dt, (Bsz, N), dev),
                                   _ptr(Dv, "Dv", f32, (D,), dev),
                                   _ptr(delta_bias, "delta_bias", f32, (D,), dev),
                                   1 if delta_softplus else 0,
                                   _ptr(z_t, "z_t", dt, (Bsz, D), dev),
                                   _ptr(out_t, "out_t", dt, (Bsz, D), dev)))
    return out_t


def ssm_decode_step(h, conv_state, x_t, W, conv_bias, delta_t, A, B_t, C_t, Dv,
                    delta_bias=None, delta_softplus=False, z_t=None, out_t=None):
    """One decode token of the block's scan branch in one launch: the conv step on x_t with
    its SiLU, then the fused scan step.  Updates h [B, D, N] and conv_state [B, K-1, D] in
    place; returns out_t [B, D]."""
    lib = load()
    Bsz, D, N = h.shape
    K = W.shape[1]
    dev = x_t.device
    dt = x_t.dtype
    code = _dtype_code(x_t)
    f32 = torch.float32
    out_t = torch.empty_like(x_t) if out_t is None else out_t
    sp = _ptr(conv_state, "conv_state", dt, (Bsz, K - 1, D), dev) if K > 1 else None
    _check(lib.ssm_decode_step(_stream(dev), code, Bsz, D, N, K,
                               _ptr(h, "h", f32, (Bsz, D, N), dev), sp,
                               _ptr(x_t, "x_t", dt, (Bsz, D), dev),
                               _ptr(W, "W", f32, (D, K), dev),
                               _ptr(conv_bias, "conv_bias", f32, (D,), dev),
                               _ptr(delta_t, "delta_t", dt, (Bsz, D), dev),
                               _ptr(A, "A", f32, (D, N), dev),
                               _ptr(B_t, "B_t", dt, (Bsz, N), dev),
                               _ptr(C_t, "C_t", dt, (Bsz, N), dev),
                               _ptr(Dv, "Dv", f32, (D,), dev),
                               _ptr(delta_bias, "delta_bias", f32, (D,), dev),
                               1 if delta_softplus else 0,
                               _ptr(z_t, "z_t", dt, (Bsz, D), dev),
                               _ptr(out_t, "out_t", dt, (Bsz, D), dev)))
    return out_t


def conv1d_causal_step(state, x_t, W, bias=None, act="none", out_t=None):
    """One token: moves the window state [B, K-1, D] in place; returns out_t [B, D]
    (silu of the conv when act="silu")."""
    lib = load()
    ac = _act_code(act)
    Bsz, D = x_t.shape
    K = W.shape[1]
    dev = x_t.device
    dt = x_t.dtype
    code = _dtype_code(x_t)
    f32 = torch.float32
    out_t = torch.empty_like(x_t) if out_t is None else out_t
    sp = _ptr(state, "state", dt, (Bsz, K - 1, D), dev) if K > 1 else None
    bp = _ptr(bias, "bias", f32, (D,), dev) if bias is not None else None
    _check(lib.conv1d_causal_step(_stream(dev), code, Bsz, D, K, sp,
                                  _ptr(x_t, "x_t", dt, (Bsz, D), dev),
                                  _ptr(W, "W", f32, (D, K), dev), bp, ac,
                                  _ptr(out_t, "out_t", dt, (Bsz, D), dev)))
    return out_t


# ----------------------------------------------------------------------------------
# sigmoid-gated scan
# ----------------------------------------------------------------------------------

def ssm_alpha_scan_fwd(a, b, Wc, h0=None, h=None):
    """h [Bn, H] = h0 + Wc x_{K-1} of the sigmoid-gated scan over a, b [Bn, K, S] (f32).
    Returns h (allocated if not given)."""
    lib = load()
    Bn, K, S = a.shape
    H = Wc.shape[0]
    dev = a.device
    f32 = torch.float32
    h = torch.empty((Bn, H), dtype=f32, device=dev) if h is None else h
    args = [_ptr(a, "a", f32, (Bn, K, S), dev), _ptr(b, "b", f32, (Bn, K, S), dev),
            _ptr(Wc, "Wc", f32, (H, S), dev), _ptr(h0, "h0", f32, (Bn, H), dev),
            _ptr(h, "h", f32, (Bn, H), dev)]
    _check(lib.ssm_alpha_scan_fwd(_stream(dev), Bn, K, S, H, *args))
    return h


def ssm_alpha_scan_bwd(a, b, Wc, dh, da=None, db=None, dWc=None, dh0=None, ws=None):
    """Backward of ssm_alpha_scan_fwd for dh [Bn, H].  dWc is accumulated into (zeros if
    not given); da, db, dh0 are overwritten.  Returns dict da, db, dWc, dh0."""
    lib = load()
    Bn, K, S = a.shape
    H = Wc.shape[0]
    dev = a.device
    f32 = torch.float32
    da = torch.empty_like(a) if da is None else da
    db = torch.empty_like(b) if db is None else db
    dWc = torch.zeros((H, S), dtype=f32, device=dev) if dWc is None else dWc
    dh0 = torch.empty((Bn, H), dtype=f32, device=dev) if dh0 is None else dh0
    args = [_ptr(a, "a", f32, (Bn, K, S), dev), _ptr(b, "b", f32, (Bn, K, S), dev),
            _ptr(Wc, "Wc", f32, (H, S), dev), _ptr(dh, "dh", f32, (Bn, H), dev),
            _ptr(da, "da", f32, (Bn, K, S), dev), _ptr(db, "db", f32, (Bn, K, S), dev),
            _ptr(dWc, "dWc", f32, (H, S), dev), _ptr(dh0, "dh0", f32, (Bn, H), dev)]
    need = int(lib.ssm_alpha_scan_bwd_workspace_bytes(Bn, K, S, H))
    ws, nbytes = _workspace(need, dev, ws)
    _check(lib.ssm_alpha_scan_bwd(_stream(dev), Bn, K, S, H, *args,
                                  _ptr(ws, "ws") if ws is not None else None, nbytes))
    return dict(da=da, db=db, dWc=dWc, dh0=dh0)
