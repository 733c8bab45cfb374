"""Python binding of libkla.so, the KLA forward scan for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/kla.h.  PyTorch supplies device
memory and the current stream.  Importing this package loads the library and
raises if it has not been built (``python bius_scan_sequence_amd/build.py``);
there is no fallback implementation.

Low-level functions carry the C names (``kla_forward``, ``kla_precision_scan``,
``kla_decode_step``, ``kla_backward``, ``kla_workspace_init``, ...) and take raw
pointers; ``forward``, ``precision_scan``, ``decode_step`` and ``backward`` are
the tensor-level helpers, and ``scan`` is the forward pass as a differentiable
torch operation (its backward calls ``backward``).
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "LIB_PATH", "lib", "KLA_F32", "KLA_BF16", "KlaError",
    "kla_forward_workspace_bytes", "kla_forward", "kla_forward_noalloc", "KLA_NOALLOC_SCRATCH_BYTES",
    "kla_forward_ou", "kla_forward_prologue", "kla_forward_vprec",
    "kla_precision_scan_workspace_bytes",
    "kla_precision_scan", "kla_decode_step", "kla_backward_workspace_bytes", "kla_backward",
    "kla_workspace_init", "kla_workspace_error", "kla_status_string", "KLA_ERR_DEVICE_WAIT", "forward", "forward_ou", "forward_prologue",
    "forward_vprec", "precision_scan",
    "decode_step", "backward", "scan", "Workspace",
]

# BIUS_KLA_LIB selects another build of the same library (the host-sanitizer
# build that tests/test_abi_sanitized.py runs the ABI tests against).
LIB_PATH = os.environ.get("BIUS_KLA_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkla.so")
KLA_F32, KLA_BF16 = 0, 1
KLA_NOALLOC_SCRATCH_BYTES = 64 << 20  # include/kla.h
# Not a C status: raised (as KlaError) when a call asked to be checked and the
# workspace's device-side error word is set (a look-back gave up waiting).
KLA_ERR_DEVICE_WAIT = 100

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python bius_scan_sequence_amd/build.py`")
lib = ctypes.CDLL(LIB_PATH)

_vp, _fp, _sz, _i = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
lib.kla_forward_workspace_bytes.restype = _sz
lib.kla_forward_workspace_bytes.argtypes = [_i] * 5
lib.kla_forward.restype = _i
lib.kla_forward.argtypes = [_vp] * 6 + [_fp] * 2 + [_vp] + [_fp] * 3 + [_i] * 6 + [_vp, _sz, _vp]
lib.kla_forward_noalloc.restype = _i
lib.kla_forward_noalloc.argtypes = [_vp] * 6 + [_fp] * 2 + [_vp] + [_fp] * 3 + [_i] * 6 + [_vp, _vp]
lib.kla_forward_ou.restype = _i
lib.kla_forward_ou.argtypes = [_vp] * 4 + [_fp] * 2 + [_vp] + [_fp] * 2 + [_vp] + [_fp] * 3 + [_i] * 6 + [_vp, _sz, _vp]
lib.kla_forward_prologue.restype = _i
lib.kla_forward_prologue.argtypes = ([_vp] * 4 + [_fp] * 2 + [_vp] + [_fp] * 6 + [_i] + [_fp] * 2 + [_vp]
                                     + [_fp] * 3 + [_i] * 6 + [_vp, _sz, _vp])
lib.kla_forward_vprec.restype = _i
lib.kla_forward_vprec.argtypes = [_vp] * 6 + [_fp] * 2 + [_vp] + [_fp] * 2 + [_i] * 6 + [_vp]
lib.kla_precision_scan_workspace_bytes.restype = _sz
lib.kla_precision_scan_workspace_bytes.argtypes = [_i] * 4
lib.kla_precision_scan.restype = _i
lib.kla_precision_scan.argtypes = [_fp] * 6 + [_i] * 4 + [_vp, _sz, _vp]
lib.kla_decode_step.restype = _i
lib.kla_decode_step.argtypes = [_vp] * 6 + [_fp] * 4 + [_vp] + [_i] * 5 + [_vp]
lib.kla_backward_workspace_bytes.restype = _sz
lib.kla_backward_workspace_bytes.argtypes = [_i] * 5
lib.kla_backward.restype = _i
lib.kla_backward.argtypes = [_vp] * 6 + [_fp] * 3 + [_vp] + [_fp] * 2 + [_vp] * 6 + [_fp] * 2 + [_i] * 6 + [_vp, _sz, _vp]
lib.kla_workspace_init.restype = _i
lib.kla_workspace_init.argtypes = [_vp, _sz, _vp]
lib.kla_workspace_error.restype = _i
lib.kla_workspace_error.argtypes = [_vp, ctypes.POINTER(ctypes.c_int), _vp]
lib.kla_status_string.restype = ctypes.c_char_p
lib.kla_status_string.argtypes = [_i]


class KlaError(RuntimeError):
    def __init__(self, code: int):
        if code == KLA_ERR_DEVICE_WAIT:
            text = "a workgroup gave up waiting for a predecessor's carry; the call's outputs are unspecified"
        else:
            text = kla_status_string(code)
        super().__init__(f"KLA status {code}: {text}")
        self.code = code


# ----------------------------------------------------------------------------- raw C ABI
def kla_forward_workspace_bytes(B, H, T, dk, dv) -> int:
    return int(lib.kla_forward_workspace_bytes(B, H, T, dk, dv))


def kla_forward(q, k, v, log_decay, proc_noise, val_prec, lambda0, M0, y, lambda_T, M_T,
                lambda_path, B, H, T, dk, dv, dtype, workspace, workspace_bytes, stream) -> int:
    return int(lib.kla_forward(q, k, v, log_decay, proc_noise, val_prec, lambda0, M0, y, lambda_T,
                               M_T, lambda_path, B, H, T, dk, dv, dtype, workspace, workspace_bytes,
                               stream))


def kla_forward_noalloc(q, k, v, log_decay, proc_noise, val_prec, lambda0, M0, y, lambda_T, M_T,
                        lambda_path, B, H, T, dk, dv, dtype, error_flag, stream) -> int:
    return int(lib.kla_forward_noalloc(q, k, v, log_decay, proc_noise, val_prec, lambda0, M0, y, lambda_T,
                                       M_T, lambda_path, B, H, T, dk, dv, dtype, error_flag, stream))


def kla_forward_ou(q, k, v, dt, theta, sigma2, val_prec, lambda0, M0, y, lambda_T, M_T, lambda_path,
                   B, H, T, dk, dv, dtype, workspace, workspace_bytes, stream) -> int:
    return int(lib.kla_forward_ou(q, k, v, dt, theta, sigma2, val_prec, lambda0, M0, y, lambda_T, M_T,
                                  lambda_path, B, H, T, dk, dv, dtype, workspace, workspace_bytes, stream))


def kla_forward_prologue(xq, xk, xv, dt_raw, theta, sigma2, vp_raw, conv_wq, conv_wk, conv_wv, conv_bq, conv_bk,
                         conv_bv, conv_width, lambda0, M0, y, lambda_T, M_T, lambda_path, B, H, T, dk, dv, dtype,
                         workspace, workspace_bytes, stream) -> int:
    return int(lib.kla_forward_prologue(xq, xk, xv, dt_raw, theta, sigma2, vp_raw, conv_wq, conv_wk, conv_wv,
                                        conv_bq, conv_bk, conv_bv, conv_width, lambda0, M0, y, lambda_T, M_T,
                                        lambda_path, B, H, T, dk, dv, dtype, workspace, workspace_bytes, stream))


def kla_forward_vprec(q, k, v, log_decay, proc_noise, val_prec, lambda0, M0, y, lambda_T, M_T,
                      B, H, T, dk, dv, dtype, stream) -> int:
    return int(lib.kla_forward_vprec(q, k, v, log_decay, proc_noise, val_prec, lambda0, M0, y, lambda_T, M_T,
                                     B, H, T, dk, dv, dtype, stream))


def kla_precision_scan_workspace_bytes(B, H, T, D) -> int:
    return int(lib.kla_precision_scan_workspace_bytes(B, H, T, D))


def kla_precision_scan(log_decay, proc_noise, obs_prec, lambda0, lambda_path, lambda_T, B, H, T, D,
                       workspace, workspace_bytes, stream) -> int:
    return int(lib.kla_precision_scan(log_decay, proc_noise, obs_prec, lambda0, lambda_path, lambda_T,
                                      B, H, T, D, workspace, workspace_bytes, stream))


def kla_decode_step(q, k, v, log_decay, proc_noise, val_prec, lambda_in, M_in, lambda_out, M_out, y,
                    B, H, dk, dv, dtype, stream) -> int:
    return int(lib.kla_decode_step(q, k, v, log_decay, proc_noise, val_prec, lambda_in, M_in, lambda_out,
                                   M_out, y, B, H, dk, dv, dtype, stream))


def kla_backward_workspace_bytes(B, H, T, dk, dv) -> int:
    return int(lib.kla_backward_workspace_bytes(B, H, T, dk, dv))


def kla_backward(q, k, v, log_decay, proc_noise, val_prec, lambda0, M0, lambda_path, grad_y, grad_lambda_T,
                 grad_M_T, grad_q, grad_k, grad_v, grad_log_decay, grad_proc_noise, grad_val_prec, grad_lambda0,
                 grad_M0, B, H, T, dk, dv, dtype, workspace, workspace_bytes, stream) -> int:
    return int(lib.kla_backward(q, k, v, log_decay, proc_noise, val_prec, lambda0, M0, lambda_path, grad_y,
                                grad_lambda_T, grad_M_T, grad_q, grad_k, grad_v, grad_log_decay, grad_proc_noise,
                                grad_val_prec, grad_lambda0, grad_M0, B, H, T, dk, dv, dtype, workspace,
                                workspace_bytes, stream))


def kla_workspace_init(workspace, workspace_bytes, stream) -> int:
    return int(lib.kla_workspace_init(workspace, workspace_bytes, stream))


def kla_workspace_error(workspace, stream=None) -> int:
    out = ctypes.c_int(0)
    rc = int(lib.kla_workspace_error(workspace, ctypes.byref(out), stream))
    if rc:
        raise KlaError(rc)
    return out.value


def kla_status_string(status: int) -> str:
    return lib.kla_status_string(status).decode()


# ----------------------------------------------------------------------------- tensors
def _torch():
    import torch
    return torch


class Workspace:
    """A zero-initialised device workspace that grows on demand.

    One workspace serves calls of ONE entry point (forward, precision_scan or
    backward) ordered on one stream: the entry points lay out their flags and
    counters differently, so they must not share a buffer.  Growing it
    allocates a new buffer and initialises it with kla_workspace_init on the
    given stream.
    """

    def __init__(self, device=None):
        torch = _torch()
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.buf = None

    def get(self, nbytes: int, stream_handle: int):
        torch = _torch()
        nbytes = max(256, (int(nbytes) + 255) // 256 * 256)
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            rc = kla_workspace_init(self.buf.data_ptr(), self.buf.numel(), stream_handle)
            if rc:
                raise KlaError(rc)
        return self.buf

    def error(self, stream_handle=None) -> int:
        """The device-side error word (see kla_workspace_error), read after the
        work queued on `stream_handle` (default: the current stream)."""
        if self.buf is None:
            return 0
        if stream_handle is None:
            stream_handle = _torch().cuda.current_stream(self.device).cuda_stream
        return kla_workspace_error(self.buf.data_ptr(), stream_handle)

    def raise_on_error(self, stream_handle=None) -> None:
        if self.error(stream_handle):
            raise KlaError(KLA_ERR_DEVICE_WAIT)


_ws_lock = threading.Lock()
_ws_cache: dict = {}


def _default_workspace(device, stream_handle, kind: str) -> Workspace:
    key = (str(device), int(stream_handle), kind)
    with _ws_lock:
        ws = _ws_cache.get(key)
        if ws is None:
            ws = _ws_cache[key] = Workspace(device)
        return ws


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check(t, name, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _outputs(out, specs, dev):
    """Preallocated outputs checked against what the call would allocate
    (shape, dtype, device, contiguity), or new tensors."""
    torch = _torch()
    if out is None:
        return tuple(torch.empty(shape, dtype=dt, device=dev) for _, shape, dt in specs)
    out = tuple(out)
    if len(out) != len(specs):
        raise ValueError(f"out holds {len(out)} tensors, expected {len(specs)}")
    for t, (name, shape, dt) in zip(out, specs):
        _check(t, f"out[{name}]", shape, dt, dev)
    return out


def _checked(ws, stream, check):
    if check:
        ws.raise_on_error(stream)


def forward(q, k, v, log_decay, proc_noise, val_prec, lambda0=None, M0=None,
            return_lambda_path=False, workspace: Workspace | None = None, out=None, check=False):
    """KLA forward pass on the current stream.

    q, k, log_decay, proc_noise, val_prec: [B,H,T,dk]; v: [B,H,T,dv]; all
    bfloat16 or all float32, contiguous, on one GPU.  lambda0 [B,H,dk] and
    M0 [B,H,dk,dv] are float32 (None: 1 and 0).  Returns
    (y [B,H,T,dv] input dtype, lambda_T [B,H,dk] f32, M_T [B,H,dk,dv] f32) and
    the f32 precision path [B,H,T,dk] when return_lambda_path.  ``out`` may
    hold preallocated (y, lambda_T, M_T) tensors (the shapes and dtypes it
    would allocate, contiguous, on the inputs' device).  With ``check`` the
    call waits for the stream and raises KlaError if a look-back gave up
    waiting (outputs unspecified); otherwise the device-side error word is
    readable through ``Workspace.error``.
    """
    torch = _torch()
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    dtype, dev = k.dtype, k.device
    if dtype == torch.bfloat16:
        code = KLA_BF16
    elif dtype == torch.float32:
        code = KLA_F32
    else:
        raise ValueError(f"unsupported dtype {dtype}")
    for name, t, shp in (("q", q, (B, H, T, dk)), ("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)),
                         ("log_decay", log_decay, (B, H, T, dk)), ("proc_noise", proc_noise, (B, H, T, dk)),
                         ("val_prec", val_prec, (B, H, T, dk))):
        _check(t, name, shp, dtype, dev)
    if lambda0 is not None:
        _check(lambda0, "lambda0", (B, H, dk), torch.float32, dev)
    if M0 is not None:
        _check(M0, "M0", (B, H, dk, dv), torch.float32, dev)
    y, lam_T, M_T = _outputs(out, (("y", (B, H, T, dv), dtype), ("lambda_T", (B, H, dk), torch.float32),
                                   ("M_T", (B, H, dk, dv), torch.float32)), dev)
    lpath = torch.empty((B, H, T, dk), dtype=torch.float32, device=dev) if return_lambda_path else None
    stream = torch.cuda.current_stream(dev).cuda_stream
    need = kla_forward_workspace_bytes(B, H, T, dk, dv)
    if need == 0:
        raise KlaError(2)
    ws_obj = workspace or _default_workspace(dev, stream, "forward")
    ws = ws_obj.get(need, stream)
    rc = kla_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(proc_noise), _ptr(val_prec),
                     _ptr(lambda0), _ptr(M0), _ptr(y), _ptr(lam_T), _ptr(M_T), _ptr(lpath),
                     B, H, T, dk, dv, code, ws.data_ptr(), ws.numel(), stream)
    if rc:
        raise KlaError(rc)
    _checked(ws_obj, stream, check)
    return (y, lam_T, M_T, lpath) if return_lambda_path else (y, lam_T, M_T)


def forward_ou(q, k, v, dt, theta, sigma2, val_prec, lambda0=None, M0=None, return_lambda_path=False,
               workspace: Workspace | None = None, out=None, check=False):
    """KLA forward pass with the OU prior in continuous time, on the current stream.

    q, k, dt, val_prec: [B,H,T,dk]; v: [B,H,T,dv] (all bfloat16 or all
    float32); theta, sigma2: float32 [H,dk], the OU rate and diffusion; the
    kernel forms log_decay = -theta dt and proc_noise = sigma2 (1 - e^{-2 theta
    dt}) / (2 theta).  Everything else as ``forward``.
    """
    torch = _torch()
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    dtype, dev = k.dtype, k.device
    code = _dtype_code(dtype)
    for name, t, shp in (("q", q, (B, H, T, dk)), ("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)),
                         ("dt", dt, (B, H, T, dk)), ("val_prec", val_prec, (B, H, T, dk))):
        _check(t, name, shp, dtype, dev)
    _check(theta, "theta", (H, dk), torch.float32, dev)
    _check(sigma2, "sigma2", (H, dk), torch.float32, dev)
    if lambda0 is not None:
        _check(lambda0, "lambda0", (B, H, dk), torch.float32, dev)
    if M0 is not None:
        _check(M0, "M0", (B, H, dk, dv), torch.float32, dev)
    y, lam_T, M_T = _outputs(out, (("y", (B, H, T, dv), dtype), ("lambda_T", (B, H, dk), torch.float32),
                                   ("M_T", (B, H, dk, dv), torch.float32)), dev)
    lpath = torch.empty((B, H, T, dk), dtype=torch.float32, device=dev) if return_lambda_path else None
    stream = torch.cuda.current_stream(dev).cuda_stream
    need = kla_forward_workspace_bytes(B, H, T, dk, dv)
    if need == 0:
        raise KlaError(2)
    ws_obj = workspace or _default_workspace(dev, stream, "forward")
    ws = ws_obj.get(need, stream)
    rc = kla_forward_ou(_ptr(q), _ptr(k), _ptr(v), _ptr(dt), _ptr(theta), _ptr(sigma2), _ptr(val_prec),
                        _ptr(lambda0), _ptr(M0), _ptr(y), _ptr(lam_T), _ptr(M_T), _ptr(lpath),
                        B, H, T, dk, dv, code, ws.data_ptr(), ws.numel(), stream)
    if rc:
        raise KlaError(rc)
    _checked(ws_obj, stream, check)
    return (y, lam_T, M_T, lpath) if return_lambda_path else (y, lam_T, M_T)


def forward_prologue(xq, xk, xv, dt_raw, theta, sigma2, vp_raw, conv_w, conv_b=(None, None, None), lambda0=None,
                     M0=None, return_lambda_path=False, workspace: Workspace | None = None, out=None, check=False):
    """KLA forward pass on raw projections, on the current stream.

    xq, xk, dt_raw, vp_raw: [B,H,T,dk]; xv: [B,H,T,dv] (all bfloat16 or all
    float32); theta, sigma2: float32 [H,dk] as ``forward_ou``; conv_w: the
    causal depthwise convolution taps of q, k, v, float32 [H,dk,W], [H,dk,W],
    [H,dv,W] (W in 1..4, tap W-1 on the current token); conv_b: their biases
    [H,d] or None.  The kernel forms q, k, v = SiLU(conv(x)) in the input
    dtype, dt = softplus(dt_raw), val_prec = softplus(vp_raw), then runs the
    scan of ``forward_ou``.  Returns as ``forward``.
    """
    torch = _torch()
    B, H, T, dk = xk.shape
    dv = xv.shape[-1]
    dtype, dev = xk.dtype, xk.device
    code = _dtype_code(dtype)
    for name, t, shp in (("xq", xq, (B, H, T, dk)), ("xk", xk, (B, H, T, dk)), ("xv", xv, (B, H, T, dv)),
                         ("dt_raw", dt_raw, (B, H, T, dk)), ("vp_raw", vp_raw, (B, H, T, dk))):
        _check(t, name, shp, dtype, dev)
    _check(theta, "theta", (H, dk), torch.float32, dev)
    _check(sigma2, "sigma2", (H, dk), torch.float32, dev)
    if len(conv_w) != 3 or len(conv_b) != 3:
        raise ValueError("conv_w and conv_b hold the (q, k, v) entries")
    W = conv_w[0].shape[-1]
    for name, t, d in (("conv_wq", conv_w[0], dk), ("conv_wk", conv_w[1], dk), ("conv_wv", conv_w[2], dv)):
        _check(t, name, (H, d, W), torch.float32, dev)
    for name, t, d in (("conv_bq", conv_b[0], dk), ("conv_bk", conv_b[1], dk), ("conv_bv", conv_b[2], dv)):
        if t is not None:
            _check(t, name, (H, d), torch.float32, dev)
    if lambda0 is not None:
        _check(lambda0, "lambda0", (B, H, dk), torch.float32, dev)
    if M0 is not None:
        _check(M0, "M0", (B, H, dk, dv), torch.float32, dev)
    y, lam_T, M_T = _outputs(out, (("y", (B, H, T, dv), dtype), ("lambda_T", (B, H, dk), torch.float32),
                                   ("M_T", (B, H, dk, dv), torch.float32)), dev)
    lpath = torch.empty((B, H, T, dk), dtype=torch.float32, device=dev) if return_lambda_path else None
    stream = torch.cuda.current_stream(dev).cuda_stream
    need = kla_forward_workspace_bytes(B, H, T, dk, dv)
    if need == 0:
        raise KlaError(2)
    ws_obj = workspace or _default_workspace(dev, stream, "forward")
    ws = ws_obj.get(need, stream)
    rc = kla_forward_prologue(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(dt_raw), _ptr(theta), _ptr(sigma2), _ptr(vp_raw),
                              *(_ptr(w) for w in conv_w), *(_ptr(b) for b in conv_b), W,
                              _ptr(lambda0), _ptr(M0), _ptr(y), _ptr(lam_T), _ptr(M_T), _ptr(lpath),
                              B, H, T, dk, dv, code, ws.data_ptr(), ws.numel(), stream)
    if rc:
        raise KlaError(rc)
    _checked(ws_obj, stream, check)
    return (y, lam_T, M_T, lpath) if return_lambda_path else (y, lam_T, M_T)


def forward_vprec(q, k, v, log_decay, proc_noise, val_prec, lambda0=None, M0=None, out=None):
    """KLA with the value precision per value channel, on the current stream.

    q, k, log_decay, proc_noise: [B,H,T,dk]; v, val_prec: [B,H,T,dv]; all
    bfloat16 or all float32.  lambda0 and M0 are float32 [B,H,dk,dv] (None: 1
    and 0).  Returns (y [B,H,T,dv] input dtype, lambda_T [B,H,dk,dv] f32,
    M_T [B,H,dk,dv] f32); ``out`` may hold preallocated tensors for them.
    """
    torch = _torch()
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    dtype, dev = k.dtype, k.device
    code = _dtype_code(dtype)
    for name, t, shp in (("q", q, (B, H, T, dk)), ("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)),
                         ("log_decay", log_decay, (B, H, T, dk)), ("proc_noise", proc_noise, (B, H, T, dk)),
                         ("val_prec", val_prec, (B, H, T, dv))):
        _check(t, name, shp, dtype, dev)
    for name, t in (("lambda0", lambda0), ("M0", M0)):
        if t is not None:
            _check(t, name, (B, H, dk, dv), torch.float32, dev)
    y, lam_T, M_T = _outputs(out, (("y", (B, H, T, dv), dtype), ("lambda_T", (B, H, dk, dv), torch.float32),
                                   ("M_T", (B, H, dk, dv), torch.float32)), dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = kla_forward_vprec(_ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(proc_noise), _ptr(val_prec),
                           _ptr(lambda0), _ptr(M0), _ptr(y), _ptr(lam_T), _ptr(M_T), B, H, T, dk, dv, code, stream)
    if rc:
        raise KlaError(rc)
    return y, lam_T, M_T


def precision_scan(log_decay, proc_noise, obs_prec, lambda0=None, workspace: Workspace | None = None,
                   out=None, check=False):
    """Precision path of B*H*D independent chains (float32 [B,H,T,D] inputs).

    Returns (lambda_path [B,H,T,D], lambda_T [B,H,D]); ``out`` may hold
    preallocated tensors for both (checked as ``forward`` checks its).
    ``check`` as ``forward``.
    """
    torch = _torch()
    B, H, T, D = log_decay.shape
    dev = log_decay.device
    for name, t in (("log_decay", log_decay), ("proc_noise", proc_noise), ("obs_prec", obs_prec)):
        _check(t, name, (B, H, T, D), torch.float32, dev)
    if lambda0 is not None:
        _check(lambda0, "lambda0", (B, H, D), torch.float32, dev)
    lpath, lam_T = _outputs(out, (("lambda_path", (B, H, T, D), torch.float32),
                                  ("lambda_T", (B, H, D), torch.float32)), dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    need = kla_precision_scan_workspace_bytes(B, H, T, D)
    if need == 0:
        raise KlaError(1)
    ws_obj = workspace or _default_workspace(dev, stream, "precision_scan")
    ws = ws_obj.get(need, stream)
    rc = kla_precision_scan(_ptr(log_decay), _ptr(proc_noise), _ptr(obs_prec), _ptr(lambda0), _ptr(lpath),
                            _ptr(lam_T), B, H, T, D, ws.data_ptr(), ws.numel(), stream)
    if rc:
        raise KlaError(rc)
    _checked(ws_obj, stream, check)
    return lpath, lam_T


def decode_step(q, k, v, log_decay, proc_noise, val_prec, lam=None, M=None, inplace=True, out=None):
    """One filter step per head on the current stream (generation, token by token).

    q, k, log_decay, proc_noise, val_prec: [B,H,dk]; v: [B,H,dv]; all bfloat16
    or all float32.  lam [B,H,dk] and M [B,H,dk,dv] are the float32 state
    before the token (None: the prior, 1 and 0).  Returns (y [B,H,dv] input
    dtype, lam_new, M_new).  With ``inplace`` (and a state given) the state
    tensors are overwritten and returned; otherwise new tensors are returned,
    or the (y, lam_new, M_new) tensors given in ``out``.
    """
    torch = _torch()
    B, H, dk = k.shape
    dv = v.shape[-1]
    dtype, dev = k.dtype, k.device
    if dtype == torch.bfloat16:
        code = KLA_BF16
    elif dtype == torch.float32:
        code = KLA_F32
    else:
        raise ValueError(f"unsupported dtype {dtype}")
    for name, t, shp in (("q", q, (B, H, dk)), ("k", k, (B, H, dk)), ("v", v, (B, H, dv)),
                         ("log_decay", log_decay, (B, H, dk)), ("proc_noise", proc_noise, (B, H, dk)),
                         ("val_prec", val_prec, (B, H, dk))):
        _check(t, name, shp, dtype, dev)
    if lam is not None:
        _check(lam, "lam", (B, H, dk), torch.float32, dev)
    if M is not None:
        _check(M, "M", (B, H, dk, dv), torch.float32, dev)
    if out is not None:
        y, lam_new, M_new = _outputs(out, (("y", (B, H, dv), dtype), ("lam_new", (B, H, dk), torch.float32),
                                           ("M_new", (B, H, dk, dv), torch.float32)), dev)
    else:
        y = torch.empty((B, H, dv), dtype=dtype, device=dev)
        lam_new = lam if (inplace and lam is not None) else torch.empty((B, H, dk), dtype=torch.float32, device=dev)
        M_new = M if (inplace and M is not None) else torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = kla_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(proc_noise), _ptr(val_prec),
                         _ptr(lam), _ptr(M), _ptr(lam_new), _ptr(M_new), _ptr(y), B, H, dk, dv, code, stream)
    if rc:
        raise KlaError(rc)
    return y, lam_new, M_new


def _dtype_code(dtype):
    torch = _torch()
    if dtype == torch.bfloat16:
        return KLA_BF16
    if dtype == torch.float32:
        return KLA_F32
    raise ValueError(f"unsupported dtype {dtype}")


def backward(q, k, v, log_decay, proc_noise, val_prec, grad_y, lambda_path, lambda0=None, M0=None,
             grad_lambda_T=None, grad_M_T=None, workspace: Workspace | None = None, out=None):
    """Gradients of the KLA forward pass on the current stream.

    Inputs as ``forward`` plus grad_y [B,H,T,dv] (input dtype), the float32
    precision path the forward call returned (``return_lambda_path=True``), and
    the optional float32 gradients of the state out, grad_lambda_T [B,H,dk]
    and grad_M_T [B,H,dk,dv].  Returns (grad_q, grad_k, grad_v,
    grad_log_decay, grad_proc_noise, grad_val_prec) in the input dtype and
    (grad_lambda0, grad_M0) in float32.  ``out`` may hold the eight
    preallocated result tensors in that order.
    """
    torch = _torch()
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    dtype, dev = k.dtype, k.device
    code = _dtype_code(dtype)
    for name, t, shp in (("q", q, (B, H, T, dk)), ("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)),
                         ("log_decay", log_decay, (B, H, T, dk)), ("proc_noise", proc_noise, (B, H, T, dk)),
                         ("val_prec", val_prec, (B, H, T, dk)), ("grad_y", grad_y, (B, H, T, dv))):
        _check(t, name, shp, dtype, dev)
    _check(lambda_path, "lambda_path", (B, H, T, dk), torch.float32, dev)
    for name, t, shp in (("lambda0", lambda0, (B, H, dk)), ("M0", M0, (B, H, dk, dv)),
                         ("grad_lambda_T", grad_lambda_T, (B, H, dk)), ("grad_M_T", grad_M_T, (B, H, dk, dv))):
        if t is not None:
            _check(t, name, shp, torch.float32, dev)
    if out is None:
        grads = [torch.empty_like(x) for x in (q, k, v, log_decay, proc_noise, val_prec)]
        g_lam0 = torch.empty((B, H, dk), dtype=torch.float32, device=dev)
        g_M0 = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    else:
        *grads, g_lam0, g_M0 = out
        for name, t, ref in zip(("grad_q", "grad_k", "grad_v", "grad_log_decay", "grad_proc_noise",
                                 "grad_val_prec"), grads, (q, k, v, log_decay, proc_noise, val_prec)):
            _check(t, name, ref.shape, dtype, dev)
        _check(g_lam0, "grad_lambda0", (B, H, dk), torch.float32, dev)
        _check(g_M0, "grad_M0", (B, H, dk, dv), torch.float32, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    need = kla_backward_workspace_bytes(B, H, T, dk, dv)
    if need == 0:
        raise KlaError(2)
    ws = (workspace or _default_workspace(dev, stream, "backward")).get(need, stream)
    rc = kla_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(proc_noise), _ptr(val_prec),
                      _ptr(lambda0), _ptr(M0), _ptr(lambda_path), _ptr(grad_y), _ptr(grad_lambda_T),
                      _ptr(grad_M_T), *(_ptr(g) for g in grads), _ptr(g_lam0), _ptr(g_M0),
                      B, H, T, dk, dv, code, ws.data_ptr(), ws.numel(), stream)
    if rc:
        raise KlaError(rc)
    return (*grads, g_lam0, g_M0)


_scan_fn = None


def _scan_function():
    global _scan_fn
    if _scan_fn is None:
        torch = _torch()

        class _Scan(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, log_decay, proc_noise, val_prec, lambda0, M0):
                y, lam_T, M_T, lpath = forward(q, k, v, log_decay, proc_noise, val_prec, lambda0, M0,
                                               return_lambda_path=True)
                ctx.ws = _default_workspace(k.device, torch.cuda.current_stream(k.device).cuda_stream, "forward")
                ctx.save_for_backward(q, k, v, log_decay, proc_noise, val_prec, lambda0, M0, lpath)
                ctx.has_state = (lambda0 is not None, M0 is not None)
                return y, lam_T, M_T

            @staticmethod
            def backward(ctx, gy, glam, gM):
                q, k, v, ld, pn, vp, lambda0, M0, lpath = ctx.saved_tensors
                gy = torch.zeros_like(v) if gy is None else gy.contiguous()
                glam = None if glam is None else glam.contiguous()
                gM = None if gM is None else gM.contiguous()
                # The precision path feeds the gradients: refuse to differentiate
                # a forward pass whose look-back gave up waiting.
                ctx.ws.raise_on_error()
                g = backward(q, k, v, ld, pn, vp, gy, lpath, lambda0, M0, glam, gM)
                return (*g[:6], g[6] if ctx.has_state[0] else None, g[7] if ctx.has_state[1] else None)

        _scan_fn = _Scan
    return _scan_fn


def scan(q, k, v, log_decay, proc_noise, val_prec, lambda0=None, M0=None):
    """The forward pass as a differentiable torch operation: returns
    (y, lambda_T, M_T) and back-propagates into every input through the
    library's backward pass."""
    return _scan_function().apply(q, k, v, log_decay, proc_noise, val_prec, lambda0, M0)
