"""ctypes binding of ``libgdn.so`` (C ABI in ``include/gdn.h``).

Argument marshalling only: checks dtype / shape / device / contiguity of the
torch tensors, passes raw device pointers, sizes and the current HIP stream,
and raises :class:`GdnError` on a non-zero status.  Every step of the method
runs in the library's kernels.  The library is loaded on first use from the
package directory; if it has not been built, that first call raises.

bf16 tensors may be ``torch.bfloat16`` or raw ``torch.int16``/``uint16`` bit
patterns; both are passed through as bits.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# GDN_LIB selects another build of the same library (e.g. a sanitizer build)
LIB_PATH = os.environ.get("GDN_LIB") or os.path.join(_HERE, "libgdn.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "gdn.h")

_lib = None

_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def lib():
    """The loaded library (ctypes.CDLL).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m linear_attention_recurrence_prep_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.gdn_version.restype = _i
        L.gdn_status_string.argtypes = [_i]
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_last_error.restype = ctypes.c_char_p
        L.gdn_recurrent.argtypes = [_p] * 8 + [_i] * 6 + [_p]
        L.gdn_recurrent.restype = _i
        L.gdn_recurrent_masked.argtypes = [_p] * 9 + [_i] * 6 + [_p]
        L.gdn_recurrent_masked.restype = _i
        L.gdn_recurrent_chunked_masked.argtypes = [_p] * 10 + [ctypes.c_size_t] + [_i] * 6 + [_p]
        L.gdn_recurrent_chunked_masked.restype = _i
        L.gdn_layer_core_masked.argtypes = [_p] * 13 + [ctypes.c_size_t] + [_i] * 7 + [_f] * 3 + [_p]
        L.gdn_layer_core_masked.restype = _i
        L.gdn_prep.argtypes = [_p] * 13 + [_i] * 7 + [_f] * 3 + [_p]
        L.gdn_prep.restype = _i
        L.gdn_recurrent_chunked.argtypes = [_p] * 9 + [ctypes.c_size_t] + [_i] * 6 + [_p]
        L.gdn_recurrent_chunked.restype = _i
        L.gdn_recurrent_chunked_workspace_bytes.argtypes = [_i] * 6
        L.gdn_recurrent_chunked_workspace_bytes.restype = ctypes.c_size_t
        L.gdn_layer_core_workspace_bytes.argtypes = [_i] * 6
        L.gdn_layer_core_workspace_bytes.restype = ctypes.c_size_t
        L.gdn_layer_core.argtypes = [_p] * 12 + [ctypes.c_size_t] + [_i] * 7 + [_f] * 3 + [_p]
        L.gdn_layer_core.restype = _i
        L.gdn_recurrent_snapshots.argtypes = [_p] * 4 + [_i] + [_p] * 6 + [_i, _p] + [_i] * 6 + [_p]
        L.gdn_recurrent_snapshots.restype = _i
        L.gdn_recurrent_per_key.argtypes = [_p] * 9 + [_i] * 6 + [_p]
        L.gdn_recurrent_per_key.restype = _i
        L.gdn_recurrent_chunked_per_key.argtypes = [_p] * 10 + [ctypes.c_size_t] + [_i] * 6 + [_p]
        L.gdn_recurrent_chunked_per_key.restype = _i
        L.gdn_recurrent_chunked_per_key_workspace_bytes.argtypes = [_i] * 6
        L.gdn_recurrent_chunked_per_key_workspace_bytes.restype = ctypes.c_size_t
        L.gdn_gated_rmsnorm.argtypes = [_p] * 4 + [_i] * 4 + [_f, _p]
        L.gdn_gated_rmsnorm.restype = _i
        L.gdn_layer_core_gated.argtypes = [_p] * 15 + [ctypes.c_size_t] + [_i] * 7 + [_f] * 4 + [_p]
        L.gdn_layer_core_gated.restype = _i
        L.gdn_layer_core_no_alloc.argtypes = [_p] * 12 + [_i] * 7 + [_f] * 3 + [_p]
        L.gdn_layer_core_no_alloc.restype = _i
        _lib = L
    return _lib


def header_functions():
    """Names of the functions declared in include/gdn.h."""
    with open(HEADER) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", text)))


def _check(status: int):
    if status != 0:
        L = lib()
        raise GdnError(status, f"{L.gdn_status_string(status).decode()}: {L.gdn_last_error().decode()}")


_capture = threading.local()


def _invoke(fn, *args):
    """Call a library entry point, or hand it to :func:`bind` when binding."""
    if getattr(_capture, "active", False):
        _capture.call = (fn, args)
        return
    _check(fn(*args))


class Bound:
    """One library call with its arguments marshalled once (see :func:`bind`)."""

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, args, keep

    def __call__(self):
        _check(self._fn(*self._args))


def bind(func, *args, **kwargs):
    """Marshal ``func(*args, **kwargs)`` (one of this module's entry points)
    once and return a zero-argument callable that issues the same library
    call again: the same kernels on the same buffers, on the stream that was
    current (or passed) at bind time, without the per-call tensor checks.
    The tensors are kept alive by the returned object; their contents may
    change between calls, their storage must not (the pointers are fixed)."""
    _capture.active = True
    _capture.call = None
    try:
        func(*args, **kwargs)
    finally:
        _capture.active = False
    if _capture.call is None:
        raise TypeError(f"{getattr(func, '__name__', func)} is not a library call of this module")
    fn, cargs = _capture.call
    _capture.call = None
    return Bound(fn, cargs, (args, kwargs))


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_MASK = (torch.uint8, torch.bool)


def _ptr(t, name, dtypes, shape, device):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.shape != shape:      # torch.Size compares equal to a tuple of the same ints
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr() if t.numel() else None


# the current stream's raw handle without building a Stream object (the
# public call is the fallback where the accessor is absent)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device, stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if _raw_stream is not None:
        return _raw_stream(device.index if device.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


def recurrent(q, k, v, g, beta, state_in, state_out, y, *, mask=None, stream=None):
    """Gated delta rule over T steps (gdn_recurrent_masked).  q,k [B,T,Hk,Dk]
    bf16; v [B,T,Hv,Dv] bf16; g,beta [B,T,Hv] f32; state_in [B,Hv,Dv,Dk] f32
    or None; state_out like state_in (may be the same tensor); y [B,T,Hv,Dv]
    bf16 (written); mask [B,T] uint8/bool or None (every step active)."""
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    dev = q.device
    args = [
        _ptr(q, "q", _BF16, (B, T, Hk, Dk), dev),
        _ptr(k, "k", _BF16, (B, T, Hk, Dk), dev),
        _ptr(v, "v", _BF16, (B, T, Hv, Dv), dev),
        _ptr(g, "g", (torch.float32,), (B, T, Hv), dev),
        _ptr(beta, "beta", (torch.float32,), (B, T, Hv), dev),
        _ptr(state_in, "state_in", (torch.float32,), (B, Hv, Dv, Dk), dev),
        _ptr(state_out, "state_out", (torch.float32,), (B, Hv, Dv, Dk), dev),
        _ptr(y, "y", _BF16, (B, T, Hv, Dv), dev),
    ]
    m = _ptr(mask, "mask", _MASK, (B, T), dev)
    _invoke(lib().gdn_recurrent_masked, *args[:5], m, *args[5:], B, T, Hk, Hv, Dk, Dv, _stream(dev, stream))


def recurrent_chunked_workspace_bytes(B, T, Hk, Hv, Dk, Dv) -> int:
    return int(lib().gdn_recurrent_chunked_workspace_bytes(B, T, Hk, Hv, Dk, Dv))


def _workspace(workspace, dev):
    if workspace is None:
        return None, 0
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    n = workspace.numel() * workspace.element_size()
    return (workspace.data_ptr() if n else None), n


def recurrent_chunked(q, k, v, g, beta, state_in, state_out, y, workspace, *, mask=None, stream=None):
    """The recurrence in 32-step chunks on the matrix cores
    (gdn_recurrent_chunked_masked).  Arguments as ``recurrent`` plus a device
    ``workspace`` tensor of at least ``recurrent_chunked_workspace_bytes``
    bytes."""
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    dev = q.device
    args = [
        _ptr(q, "q", _BF16, (B, T, Hk, Dk), dev),
        _ptr(k, "k", _BF16, (B, T, Hk, Dk), dev),
        _ptr(v, "v", _BF16, (B, T, Hv, Dv), dev),
        _ptr(g, "g", (torch.float32,), (B, T, Hv), dev),
        _ptr(beta, "beta", (torch.float32,), (B, T, Hv), dev),
        _ptr(state_in, "state_in", (torch.float32,), (B, Hv, Dv, Dk), dev),
        _ptr(state_out, "state_out", (torch.float32,), (B, Hv, Dv, Dk), dev),
        _ptr(y, "y", _BF16, (B, T, Hv, Dv), dev),
    ]
    ws, nws = _workspace(workspace, dev)
    m = _ptr(mask, "mask", _MASK, (B, T), dev)
    _invoke(lib().gdn_recurrent_chunked_masked, *args[:5], m, *args[5:], ws, nws, B, T, Hk, Hv, Dk, Dv,
            _stream(dev, stream))


def prep(qkv, conv_w, conv_state_in, conv_state_out, a, b, A_log, dt_bias, q, k, v, g, beta, *,
         Hk, Hv, Dk, Dv, q_scale, k_scale, eps=1e-6, stream=None):
    """Prologue (gdn_prep).  qkv [B,T,C] bf16, conv_w [C,K] bf16,
    conv_state_in/out [B,K-1,C] bf16 or None, a,b [B,T,Hv] bf16, A_log,
    dt_bias [Hv] f32; outputs q,k [B,T,Hk,Dk] bf16, v [B,T,Hv,Dv] bf16,
    g,beta [B,T,Hv] f32."""
    B, T, C = qkv.shape
    K = conv_w.shape[1]
    dev = qkv.device
    args = [
        _ptr(qkv, "qkv", _BF16, (B, T, C), dev),
        _ptr(conv_w, "conv_w", _BF16, (C, K), dev),
        _ptr(conv_state_in, "conv_state_in", _BF16, (B, K - 1, C), dev),
        _ptr(conv_state_out, "conv_state_out", _BF16, (B, K - 1, C), dev),
        _ptr(a, "a", _BF16, (B, T, Hv), dev),
        _ptr(b, "b", _BF16, (B, T, Hv), dev),
        _ptr(A_log, "A_log", (torch.float32,), (Hv,), dev),
        _ptr(dt_bias, "dt_bias", (torch.float32,), (Hv,), dev),
        _ptr(q, "q", _BF16, (B, T, Hk, Dk), dev),
        _ptr(k, "k", _BF16, (B, T, Hk, Dk), dev),
        _ptr(v, "v", _BF16, (B, T, Hv, Dv), dev),
        _ptr(g, "g", (torch.float32,), (B, T, Hv), dev),
        _ptr(beta, "beta", (torch.float32,), (B, T, Hv), dev),
    ]
    _invoke(lib().gdn_prep, *args, B, T, Hk, Hv, Dk, Dv, K, q_scale, k_scale, eps,
            _stream(dev, stream))


def layer_core_workspace_bytes(B, T, Hk, Hv, Dk, Dv) -> int:
    return int(lib().gdn_layer_core_workspace_bytes(B, T, Hk, Hv, Dk, Dv))


def layer_core(qkv, conv_w, conv_state_in, conv_state_out, a, b, A_log, dt_bias,
               state_in, state_out, y, workspace, *, Hk, Hv, Dk, Dv, q_scale, k_scale,
               eps=1e-6, mask=None, stream=None):
    """Prologue then recurrence (gdn_layer_core_masked).  Arguments as
    ``prep`` and ``recurrent``; ``workspace`` is a uint8/int8 device tensor of
    at least ``layer_core_workspace_bytes(...)`` bytes (or None when that is
    0); ``mask`` [B,T] masks recurrence steps (None = all active)."""
    B, T, C = qkv.shape
    K = conv_w.shape[1]
    dev = qkv.device
    ws_ptr, ws_bytes = _workspace(workspace, dev)
    args = [
        _ptr(qkv, "qkv", _BF16, (B, T, C), dev),
        _ptr(conv_w, "conv_w", _BF16, (C, K), dev),
        _ptr(conv_state_in, "conv_state_in", _BF16, (B, K - 1, C), dev),
        _ptr(conv_state_out, "conv_state_out", _BF16, (B, K - 1, C), dev),
        _ptr(a, "a", _BF16, (B, T, Hv), dev),
        _ptr(b, "b", _BF16, (B, T, Hv), dev),
        _ptr(A_log, "A_log", (torch.float32,), (Hv,), dev),
        _ptr(dt_bias, "dt_bias", (torch.float32,), (Hv,), dev),
        _ptr(state_in, "state_in", (torch.float32,), (B, Hv, Dv, Dk), dev),
        _ptr(state_out, "state_out", (torch.float32,), (B, Hv, Dv, Dk), dev),
        _ptr(y, "y", _BF16, (B, T, Hv, Dv), dev),
        ws_ptr,
    ]
    m = _ptr(mask, "mask", _MASK, (B, T), dev)
    _invoke(lib().gdn_layer_core_masked, *args[:8], m, *args[8:], ws_bytes, B, T, Hk, Hv, Dk, Dv, K, q_scale,
            k_scale, eps, _stream(dev, stream))


# workspace bytes held by the library for layer_core_no_alloc (the header's
# GDN_NO_ALLOC_SCRATCH_BYTES)
NO_ALLOC_SCRATCH_BYTES = 128 << 20


def layer_core_no_alloc(qkv, conv_w, conv_state_in, conv_state_out, a, b, A_log, dt_bias,
                        state_in, state_out, y, *, Hk, Hv, Dk, Dv, q_scale, k_scale,
                        eps=1e-6, mask=None, stream=None):
    """The layer core with the library's own device scratch as its workspace
    (gdn_layer_core_no_alloc): arguments as ``layer_core`` without
    ``workspace``; sizes whose workspace exceeds NO_ALLOC_SCRATCH_BYTES raise.
    Calls that can overlap in time on one device race on that scratch."""
    B, T, C = qkv.shape
    K = conv_w.shape[1]
    dev = qkv.device
    args = [
        _ptr(qkv, "qkv", _BF16, (B, T, C), dev),
        _ptr(conv_w, "conv_w", _BF16, (C, K), dev),
        _ptr(conv_state_in, "conv_state_in", _BF16, (B, K - 1, C), dev),
        _ptr(conv_state_out, "conv_state_out", _BF16, (B, K - 1, C), dev),
        _ptr(a, "a", _BF16, (B, T, Hv), dev),
        _ptr(b, "b", _BF16, (B, T, Hv), dev),
        _ptr(A_log, "A_log", (torch.float32,), (Hv,), dev),
        _ptr(dt_bias, "dt_bias", (torch.float32,), (Hv,), dev),
        _ptr(mask, "mask", _MASK, (B, T), dev),
        _ptr(state_in, "state_in", (torch.float32,), (B, Hv, Dv, Dk), dev),
        _ptr(state_out, "state_out", (torch.float32,), (B, Hv, Dv, Dk), dev),
        _ptr(y, "y", _BF16, (B, T, Hv, Dv), dev),
    ]
    _invoke(lib().gdn_layer_core_no_alloc, *args, B, T, Hk, Hv, Dk, Dv, K, q_scale, k_scale, eps,
            _stream(dev, stream))


def gated_rmsnorm(y, z, norm_weight, out, *, eps=1e-6, stream=None):
    """Output epilogue (gdn_gated_rmsnorm): out = bf16(silu(z) * rms_norm(y)
    * norm_weight) per row of Dv.  y, z, out [B,T,Hv,Dv] bf16 (out may be y
    or z itself); norm_weight [Dv] bf16."""
    B, T, Hv, Dv = y.shape
    dev = y.device
    args = [
        _ptr(y, "y", _BF16, (B, T, Hv, Dv), dev),
        _ptr(z, "z", _BF16, (B, T, Hv, Dv), dev),
        _ptr(norm_weight, "norm_weight", _BF16, (Dv,), dev),
        _ptr(out, "out", _BF16, (B, T, Hv, Dv), dev),
    ]
    _invoke(lib().gdn_gated_rmsnorm, *args, B, T, Hv, Dv, eps, _stream(dev, stream))


def layer_core_gated(qkv, conv_w, conv_state_in, conv_state_out, a, b, A_log, dt_bias, z, norm_weight,
                     state_in, state_out, out, workspace, *, Hk, Hv, Dk, Dv, q_scale, k_scale,
                     eps=1e-6, norm_eps=1e-6, mask=None, stream=None):
    """Layer core then the output epilogue (gdn_layer_core_gated).  Arguments
    as ``layer_core`` plus z [B,T,Hv,Dv] and norm_weight [Dv] (bf16); ``out``
    [B,T,Hv,Dv] bf16 receives silu(z)·rms_norm(y)·norm_weight."""
    B, T, C = qkv.shape
    K = conv_w.shape[1]
    dev = qkv.device
    ws_ptr, ws_bytes = _workspace(workspace, dev)
    args = [
        _ptr(qkv, "qkv", _BF16, (B, T, C), dev),
        _ptr(conv_w, "conv_w", _BF16, (C, K), dev),
        _ptr(conv_state_in, "conv_state_in", _BF16, (B, K - 1, C), dev),
        _ptr(conv_state_out, "conv_state_out", _BF16, (B, K - 1, C), dev),
        _ptr(a, "a", _BF16, (B, T, Hv), dev),
        _ptr(b, "b", _BF16, (B, T, Hv), dev),
        _ptr(A_log, "A_log", (torch.float32,), (Hv,), dev),
        _ptr(dt_bias, "dt_bias", (torch.float32,), (Hv,), dev),
        _ptr(z, "z", _BF16, (B, T, Hv, Dv), dev),
        _ptr(norm_weight, "norm_weight", _BF16, (Dv,), dev),
        _ptr(mask, "mask", _MASK, (B, T), dev),
        _ptr(state_in, "state_in", (torch.float32,), (B, Hv, Dv, Dk), dev),
        _ptr(state_out, "state_out", (torch.float32,), (B, Hv, Dv, Dk), dev),
        _ptr(out, "out", _BF16, (B, T, Hv, Dv), dev),
        ws_ptr,
    ]
    _invoke(lib().gdn_layer_core_gated, *args, ws_bytes, B, T, Hk, Hv, Dk, Dv, K, q_scale, k_scale, eps,
            norm_eps, _stream(dev, stream))


def recurrent_snapshots(q, k, v, g, beta, state_in, state_out, y, snap_steps, snapshots, *, mask=None,
                        stream=None):
    """The recurrence (per-step form) that also writes the state after each
    step count in ``snap_steps`` (a list of strictly increasing ints in
    [0, T], at most 32) into ``snapshots`` [n, B, Hv, Dv, Dk] f32
    (gdn_recurrent_snapshots).  ``g`` is [B,T,Hv] (per-head decay) or
    [B,T,Hv,Dk] (per-key decay); other arguments as ``recurrent``."""
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    dev = q.device
    per_key = g is not None and g.dim() == 4
    steps = [int(s_) for s_ in snap_steps]
    arr = (ctypes.c_int32 * max(len(steps), 1))(*steps)
    args = [
        _ptr(q, "q", _BF16, (B, T, Hk, Dk), dev),
        _ptr(k, "k", _BF16, (B, T, Hk, Dk), dev),
        _ptr(v, "v", _BF16, (B, T, Hv, Dv), dev),
        _ptr(g, "g", (torch.float32,), (B, T, Hv, Dk) if per_key else (B, T, Hv), dev),
    ]
    rest = [
        _ptr(beta, "beta", (torch.float32,), (B, T, Hv), dev),
        _ptr(mask, "mask", _MASK, (B, T), dev),
        _ptr(state_in, "state_in", (torch.float32,), (B, Hv, Dv, Dk), dev),
        _ptr(state_out, "state_out", (torch.float32,), (B, Hv, Dv, Dk), dev),
        _ptr(y, "y", _BF16, (B, T, Hv, Dv), dev),
    ]
    snaps = _ptr(snapshots, "snapshots", (torch.float32,), (len(steps), B, Hv, Dv, Dk), dev)
    _invoke(lib().gdn_recurrent_snapshots, *args, int(per_key), *rest, ctypes.cast(arr, ctypes.c_void_p),
            len(steps), snaps, B, T, Hk, Hv, Dk, Dv, _stream(dev, stream))


def recurrent_per_key(q, k, v, g, beta, state_in, state_out, y, *, mask=None, stream=None):
    """The recurrence with the per-key decay gate g [B,T,Hv,Dk] f32
    (gdn_recurrent_per_key); other arguments as ``recurrent``."""
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    dev = q.device
    args = [
        _ptr(q, "q", _BF16, (B, T, Hk, Dk), dev),
        _ptr(k, "k", _BF16, (B, T, Hk, Dk), dev),
        _ptr(v, "v", _BF16, (B, T, Hv, Dv), dev),
        _ptr(g, "g", (torch.float32,), (B, T, Hv, Dk), dev),
        _ptr(beta, "beta", (torch.float32,), (B, T, Hv), dev),
        _ptr(mask, "mask", _MASK, (B, T), dev),
        _ptr(state_in, "state_in", (torch.float32,), (B, Hv, Dv, Dk), dev),
        _ptr(state_out, "state_out", (torch.float32,), (B, Hv, Dv, Dk), dev),
        _ptr(y, "y", _BF16, (B, T, Hv, Dv), dev),
    ]
    _invoke(lib().gdn_recurrent_per_key, *args, B, T, Hk, Hv, Dk, Dv, _stream(dev, stream))


def recurrent_chunked_per_key_workspace_bytes(B, T, Hk, Hv, Dk, Dv) -> int:
    return int(lib().gdn_recurrent_chunked_per_key_workspace_bytes(B, T, Hk, Hv, Dk, Dv))


def recurrent_chunked_per_key(q, k, v, g, beta, state_in, state_out, y, workspace, *, mask=None, stream=None):
    """The recurrence with the per-key decay gate g [B,T,Hv,Dk] f32 in 32-step
    chunks on the matrix cores (gdn_recurrent_chunked_per_key).  Arguments as
    ``recurrent_per_key`` plus a device ``workspace`` tensor of at least
    ``recurrent_chunked_per_key_workspace_bytes`` bytes."""
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    dev = q.device
    args = [
        _ptr(q, "q", _BF16, (B, T, Hk, Dk), dev),
        _ptr(k, "k", _BF16, (B, T, Hk, Dk), dev),
        _ptr(v, "v", _BF16, (B, T, Hv, Dv), dev),
        _ptr(g, "g", (torch.float32,), (B, T, Hv, Dk), dev),
        _ptr(beta, "beta", (torch.float32,), (B, T, Hv), dev),
        _ptr(mask, "mask", _MASK, (B, T), dev),
        _ptr(state_in, "state_in", (torch.float32,), (B, Hv, Dv, Dk), dev),
        _ptr(state_out, "state_out", (torch.float32,), (B, Hv, Dv, Dk), dev),
        _ptr(y, "y", _BF16, (B, T, Hv, Dv), dev),
    ]
    ws, nws = _workspace(workspace, dev)
    _invoke(lib().gdn_recurrent_chunked_per_key, *args, ws, nws, B, T, Hk, Hv, Dk, Dv, _stream(dev, stream))
