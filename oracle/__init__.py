"""CPU oracle for the Gated DeltaNet layer core -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It never imports the HIP library and
the HIP library never imports it; they share no code.

The arithmetic lives in ``gdn_oracle.c`` (plain single-threaded fp64 C, one
rounding per operation, loops in the pages' order).  This module only loads
that library with ctypes, marshals numpy arrays, and converts between stored
formats:

* ``bf16`` tensors are numpy ``uint16`` arrays of raw bit patterns;
* the oracle's outputs are ``float64`` (unrounded), except the conv-state
  tail, which is an exact bf16 copy.

Sources: "mlex 0.1.2 -- src/models/gated_delta.rs" (GatedDeltaNet::forward)
and "mlx-bun 0.4.0 -> 1.0.0, package/src/model/qwen3-delta.ts" (layout and
dtype contract in the file header, compute_g, gated_delta_step).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB, build

_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_hp = ctypes.POINTER(ctypes.c_uint16)
_bp = ctypes.POINTER(ctypes.c_uint8)
_i = ctypes.c_int
_d = ctypes.c_double


def lib():
    """Load (building first if absent) the oracle's shared library."""
    global _lib
    if _lib is None:
        # GDN_ORACLE_LIB selects another build of the oracle (a sanitizer build)
        path = os.environ.get("GDN_ORACLE_LIB")
        if path is None:
            path = LIB
            if not os.path.exists(path):
                build()
        L = ctypes.CDLL(path)
        L.oracle_f64_to_bf16.argtypes = [_d]
        L.oracle_f64_to_bf16.restype = ctypes.c_uint16
        L.oracle_round_bf16_array.argtypes = [_dp, _hp, ctypes.c_size_t]
        L.oracle_round_bf16_array.restype = None
        L.oracle_bf16_to_f64_array.argtypes = [_hp, _dp, ctypes.c_size_t]
        L.oracle_bf16_to_f64_array.restype = None
        L.oracle_prep.argtypes = [_hp, _hp, _hp, _hp, _hp, _hp, _fp, _fp,
                                  _dp, _dp, _dp, _dp, _dp,
                                  _i, _i, _i, _i, _i, _i, _i, _d, _d, _d]
        L.oracle_prep.restype = _i
        L.oracle_recurrent.argtypes = [_dp, _dp, _dp, _dp, _dp, _bp, _dp, _dp, _dp,
                                       _i, _i, _i, _i, _i, _i]
        L.oracle_recurrent.restype = _i
        L.oracle_recurrent_per_key.argtypes = L.oracle_recurrent.argtypes
        L.oracle_recurrent_per_key.restype = _i
        L.oracle_layer_core.argtypes = [_hp, _hp, _hp, _hp, _hp, _hp, _fp, _fp, _bp,
                                        _dp, _dp, _dp,
                                        _i, _i, _i, _i, _i, _i, _i, _d, _d, _d]
        L.oracle_layer_core.restype = _i
        L.oracle_gated_rmsnorm.argtypes = [_hp, _hp, _hp, _dp, ctypes.c_long, _i, _d]
        L.oracle_gated_rmsnorm.restype = _i
        L.oracle_rms_scale.argtypes = [_dp, _dp, ctypes.c_long, _i, _d, _d]
        L.oracle_rms_scale.restype = None
        L.oracle_gates.argtypes = [_hp, _hp, _fp, _fp, _dp, _dp, ctypes.c_long, _i]
        L.oracle_gates.restype = None
        _lib = L
    return _lib


def _ptr(a, typ):
    if a is None:
        return ctypes.cast(None, typ)
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(typ)


def _h(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _f32(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.float32, a.dtype
    return a


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _mask(a):
    """Step mask as contiguous bytes (nonzero = active), or None."""
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a) != 0, dtype=np.uint8)


# ------------------------------------------------------------------ formats

def round_bf16(x) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_round_bf16_array(_ptr(x, _dp), _ptr(out, _hp), x.size)
    return out


def bf16_to_f64(h) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    h = _h(h)
    out = np.empty(h.shape, dtype=np.float64)
    lib().oracle_bf16_to_f64_array(_ptr(h, _hp), _ptr(out, _dp), h.size)
    return out


def round_f32(x) -> np.ndarray:
    """Round float64 values to float32 (nearest, ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


# ---------------------------------------------------------------- the method

def prep(qkv, conv_w, conv_state_in, a, b, A_log, dt_bias, *, Hk, Hv, Dk, Dv,
         q_scale, k_scale, eps=1e-6):
    """Prologue in fp64.  Shapes: qkv [B,T,C], conv_w [C,K], conv_state_in
    [B,K-1,C] or None, a/b [B,T,Hv] (all bf16 bits); A_log, dt_bias [Hv] f32.

    Returns dict(q, k [B,T,Hk,Dk], v [B,T,Hv,Dv], g, beta [B,T,Hv]: float64
    unrounded; conv_state [B,K-1,C] bf16 bits)."""
    qkv, conv_w, conv_state_in, a, b = map(_h, (qkv, conv_w, conv_state_in, a, b))
    A_log, dt_bias = _f32(A_log), _f32(dt_bias)
    B, T, C = qkv.shape
    K = conv_w.shape[1]
    assert C == 2 * Hk * Dk + Hv * Dv and conv_w.shape == (C, K)
    assert a.shape == (B, T, Hv) and b.shape == (B, T, Hv)
    if conv_state_in is not None:
        assert conv_state_in.shape == (B, K - 1, C)
    q = np.empty((B, T, Hk, Dk))
    k = np.empty((B, T, Hk, Dk))
    v = np.empty((B, T, Hv, Dv))
    g = np.empty((B, T, Hv))
    beta = np.empty((B, T, Hv))
    cs = np.empty((B, K - 1, C), dtype=np.uint16)
    rc = lib().oracle_prep(_ptr(qkv, _hp), _ptr(conv_w, _hp), _ptr(conv_state_in, _hp),
                           _ptr(cs, _hp), _ptr(a, _hp), _ptr(b, _hp),
                           _ptr(A_log, _fp), _ptr(dt_bias, _fp),
                           _ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(g, _dp),
                           _ptr(beta, _dp), B, T, Hk, Hv, Dk, Dv, K,
                           float(q_scale), float(k_scale), float(eps))
    if rc != 0:
        raise RuntimeError("oracle_prep failed")
    return dict(q=q, k=k, v=v, g=g, beta=beta, conv_state=cs)


def recurrent(q, k, v, g, beta, state_in=None, mask=None):
    """Gated delta rule in fp64.  q,k [B,T,Hk,Dk]; v [B,T,Hv,Dv]; g [B,T,Hv]
    (per-head decay) or [B,T,Hv,Dk] (per-key decay); beta [B,T,Hv];
    state_in [B,Hv,Dv,Dk] or None; mask [B,T] (nonzero = active step) or
    None.  Inputs are taken as exact values (widened to float64).  Returns
    (y [B,T,Hv,Dv], state_out)."""
    q, k, v, g, beta, state_in = map(_f64, (q, k, v, g, beta, state_in))
    mask = _mask(mask)
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    assert k.shape == q.shape and v.shape[:2] == (B, T)
    per_key = g.ndim == 4
    assert g.shape == ((B, T, Hv, Dk) if per_key else (B, T, Hv)) and beta.shape == (B, T, Hv)
    if state_in is not None:
        assert state_in.shape == (B, Hv, Dv, Dk)
    y = np.empty((B, T, Hv, Dv))
    s = np.empty((B, Hv, Dv, Dk))
    if mask is not None:
        assert mask.shape == (B, T)
    fn = lib().oracle_recurrent_per_key if per_key else lib().oracle_recurrent
    rc = fn(_ptr(q, _dp), _ptr(k, _dp), _ptr(v, _dp), _ptr(g, _dp),
                                _ptr(beta, _dp), _ptr(mask, _bp), _ptr(state_in, _dp), _ptr(s, _dp),
                                _ptr(y, _dp), B, T, Hk, Hv, Dk, Dv)
    if rc != 0:
        raise RuntimeError("oracle_recurrent failed")
    return y, s


def recurrent_snapshots(q, k, v, g, beta, steps, state_in=None, mask=None):
    """States after the first n steps, for each n in ``steps``: the
    recurrence run over each prefix of the inputs.  Returns
    [len(steps), B, Hv, Dv, Dk] float64."""
    out = []
    for n in steps:
        sl = lambda a: None if a is None else np.ascontiguousarray(np.asarray(a)[:, :n])
        _, s = recurrent(sl(q), sl(k), sl(v), sl(g), sl(beta), state_in, sl(mask))
        out.append(s)
    return np.stack(out)


def layer_core(qkv, conv_w, conv_state_in, a, b, A_log, dt_bias, state_in=None, *,
               Hk, Hv, Dk, Dv, q_scale, k_scale, eps=1e-6, mask=None):
    """Prologue, stored-dtype roundings (q,k,v -> bf16; g,beta -> f32), then
    the recurrence (mask [B,T] masks recurrence steps, None = all active).
    Returns (y float64 [B,T,Hv,Dv], state_out float64, conv_state_out bf16
    bits)."""
    qkv, conv_w, conv_state_in, a, b = map(_h, (qkv, conv_w, conv_state_in, a, b))
    mask = _mask(mask)
    A_log, dt_bias = _f32(A_log), _f32(dt_bias)
    state_in = _f64(state_in)
    B, T, C = qkv.shape
    K = conv_w.shape[1]
    assert C == 2 * Hk * Dk + Hv * Dv and conv_w.shape == (C, K)
    if state_in is not None:
        assert state_in.shape == (B, Hv, Dv, Dk)
    y = np.empty((B, T, Hv, Dv))
    s = np.empty((B, Hv, Dv, Dk))
    cs = np.empty((B, K - 1, C), dtype=np.uint16)
    rc = lib().oracle_layer_core(_ptr(qkv, _hp), _ptr(conv_w, _hp), _ptr(conv_state_in, _hp),
                                 _ptr(cs, _hp), _ptr(a, _hp), _ptr(b, _hp),
                                 _ptr(A_log, _fp), _ptr(dt_bias, _fp), _ptr(mask, _bp),
                                 _ptr(state_in, _dp), _ptr(s, _dp), _ptr(y, _dp),
                                 B, T, Hk, Hv, Dk, Dv, K,
                                 float(q_scale), float(k_scale), float(eps))
    if rc != 0:
        raise RuntimeError("oracle_layer_core failed")
    return y, s, cs


def gated_rmsnorm(y, z, norm_weight, eps=1e-6):
    """Output epilogue in fp64: silu(z) * rms_norm(y) * norm_weight per row of
    Dv values, from stored bf16 bits y, z [..., Dv] and norm_weight [Dv].
    Returns float64 of y's shape (round_bf16 gives the stored result)."""
    y, z, w = _h(y), _h(z), _h(norm_weight)
    Dv = y.shape[-1]
    assert z.shape == y.shape and w.shape == (Dv,)
    out = np.empty(y.shape)
    rc = lib().oracle_gated_rmsnorm(_ptr(y, _hp), _ptr(z, _hp), _ptr(w, _hp), _ptr(out, _dp),
                                    y.size // Dv, Dv, float(eps))
    if rc != 0:
        raise RuntimeError("oracle_gated_rmsnorm failed")
    return out


def rms_scale(x, scale, eps=1e-6):
    """x / sqrt(mean(x^2) + eps) * scale over the last axis, in fp64
    (the C routine the prologue uses for q and k)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    D = x.shape[-1]
    out = np.empty_like(x)
    lib().oracle_rms_scale(_ptr(x, _dp), _ptr(out, _dp), x.size // D, D,
                           float(scale), float(eps))
    return out


def gates(a, b, A_log, dt_bias):
    """(g, beta) in fp64 from stored a, b [..., Hv] bf16 bits and per-head
    A_log, dt_bias [Hv] f32 (the C routine the prologue uses)."""
    a, b = _h(a), _h(b)
    A_log, dt_bias = _f32(A_log), _f32(dt_bias)
    assert a.shape == b.shape
    Hv = a.shape[-1]
    assert A_log.shape == (Hv,) and dt_bias.shape == (Hv,)
    g = np.empty(a.shape)
    beta = np.empty(a.shape)
    lib().oracle_gates(_ptr(a, _hp), _ptr(b, _hp), _ptr(A_log, _fp), _ptr(dt_bias, _fp),
                       _ptr(g, _dp), _ptr(beta, _dp), a.size // Hv, Hv)
    return g, beta


def recurrence_inputs(raw, *, q_scale=None, k_scale=None, eps=1e-6):
    """Stored recurrence inputs for the recurrence-only workloads, derived
    from raw draws: q and k RMS-normalised over Dk and scaled (default
    Dk^-1/2 for both), g and beta from a, b, A_log, dt_bias; then q, k, v in
    bf16 and g, beta in f32 -- the dtypes the recurrence receives.

    ``raw``: q_raw, k_raw [B,T,Hk,Dk], v [B,T,Hv,Dv], a, b [B,T,Hv] as bf16
    bits; A_log, dt_bias [Hv] f32.  Returns dict(q, k, v: bf16 bits; g, beta:
    float32)."""
    Dk = raw["q_raw"].shape[-1]
    if q_scale is None:
        q_scale = Dk ** -0.5
    if k_scale is None:
        k_scale = Dk ** -0.5
    qn = rms_scale(bf16_to_f64(raw["q_raw"]), q_scale, eps)
    kn = rms_scale(bf16_to_f64(raw["k_raw"]), k_scale, eps)
    g, beta = gates(raw["a"], raw["b"], raw["A_log"], raw["dt_bias"])
    return dict(q=round_bf16(qn), k=round_bf16(kn), v=np.ascontiguousarray(raw["v"]),
                g=round_f32(g), beta=round_f32(beta))
