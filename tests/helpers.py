"""Shared helpers for the parity tests: device transfer of bf16 bit patterns,
the tolerances, and oracle sub-problem slicing."""
from __future__ import annotations

import math

import sys

import numpy as np
import torch

import oracle

DEV = "cuda:0"
U32 = 2.0 ** -24          # unit roundoff of binary32


def to_dev(a, device=DEV):
    """numpy uint16 bf16 bits / float32 -> torch tensor on the device."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device)
    assert a.dtype == np.float32, a.dtype
    return torch.from_numpy(a).to(device)


def bits(t):
    """bf16/int16 tensor -> numpy uint16 bit patterns."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f32(t):
    return t.detach().cpu().numpy()


def bf16_ulp(x):
    """Spacing of bf16 values at |x| (subnormal spacing below 2^-126)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.where(ax > 0, np.maximum(e, -126), -126)
    return np.exp2(e - 7)


# y against the fp64 reference, per (b, v-head).  Beside the stated bound
# (1 bf16 ulp + 1e-3 absolute), which does not bind where |y| is far below
# 1e-3, two bounds that do:
#   |dy| <= ulp(y_ref) + Y_HEAD_TOL * max|y_ref| over the head, elementwise;
#   at most 1 ulp from y_ref where |y_ref| >= Y_ULP_FLOOR * max|y_ref|.
# The device rounds an f32 value to bf16 (half an ulp) whose own error is a
# few units of 2^-16 (chunked form: the leading two planes of the y path) or
# of 2^-24 * Dk (per-step form) times the size of the terms, which are of the
# order of the head's largest outputs; so Y_HEAD_TOL leaves a margin of 16
# over the chunked form's truncation, and above Y_ULP_FLOOR the pre-rounding
# error is below a quarter of an ulp.  y = 0, or a 1 % error in any output
# above 2^-5 of its head's largest, fails both.
Y_HEAD_TOL = 2.0 ** -12
Y_ULP_FLOOR = 2.0 ** -4


def _head_max(y_ref):
    """max |y_ref| per (b, v-head) of a [B, T, Hv, Dv] array, broadcastable."""
    return np.abs(y_ref).max(axis=(1, 3), keepdims=True) if y_ref.size else np.zeros((1, 1, 1, 1))


def check_y(y_bits, y_ref, label="", strict=True):
    """y (bf16 bits [B,T,Hv,Dv]) against the fp64 reference.  Always: within 1
    bf16 ulp + 1e-3 absolute.  strict: also the per-head bounds above (the
    reference must then be the recurrence on the very inputs the device used).
    Returns the observed figures."""
    y = oracle.bf16_to_f64(y_bits)
    assert not np.isnan(y).any(), f"{label}: NaN in y"
    err = np.abs(y - y_ref)
    ulp = bf16_ulp(y_ref)
    bad = err > ulp + 1e-3
    assert not bad.any(), (f"{label}: {bad.sum()} y elements beyond 1 ulp + 1e-3; worst err "
                           f"{err.max():.3e}")
    out = dict(max_abs=float(err.max()) if err.size else 0.0,
               max_ulp=float((err / ulp).max()) if err.size else 0.0)
    if not strict or not err.size:
        return out
    hm = _head_max(y_ref)
    rel = err / np.maximum(hm, 1e-300)
    bad = err > ulp + Y_HEAD_TOL * hm
    assert not bad.any(), (f"{label}: {bad.sum()} y elements beyond 1 ulp + 2^-12 of the head's largest; "
                           f"worst {rel.max():.3e} of it")
    big = np.abs(y_ref) >= Y_ULP_FLOOR * hm
    ulps_big = float((err / ulp)[big].max()) if big.any() else 0.0
    assert ulps_big <= 1.0, f"{label}: y {ulps_big:.2f} ulp from the reference where |y| >= 2^-4 of its head's max"
    out.update(head_rel=float(rel.max()), max_ulp_big=ulps_big)
    return out


def state_err(s_gpu, s_ref):
    """Per-head normwise error max_{b,hv} ||dS||_inf / ||S_ref||_inf."""
    d = np.abs(s_gpu.astype(np.float64) - s_ref).reshape(s_ref.shape[0], s_ref.shape[1], -1).max(-1)
    n = np.abs(s_ref).reshape(s_ref.shape[0], s_ref.shape[1], -1).max(-1)
    return float(np.max(d / np.maximum(n, 1e-300))) if d.size else 0.0


def state_err_elementwise(s_gpu, s_ref, floor=1e-3):
    """For information only: the largest elementwise relative error over the
    entries with |S_ref| >= floor * max |S_ref| of their (b, v-head) (the
    elementwise ratio is unbounded at entries near zero, so it is not a
    tolerance)."""
    ref = s_ref.reshape(s_ref.shape[0], s_ref.shape[1], -1)
    d = np.abs(s_gpu.astype(np.float64).reshape(ref.shape) - ref)
    n = np.abs(ref).max(-1, keepdims=True)
    big = (np.abs(ref) >= floor * n) & (ref != 0)     # (an all-zero head has no such entries)
    return float((d[big] / np.abs(ref[big])).max()) if big.any() else 0.0


def check_state(s_gpu, s_ref, tol, label=""):
    assert not np.isnan(s_gpu).any(), f"{label}: NaN in state"
    e = state_err(s_gpu, s_ref)
    assert e <= tol, f"{label}: state normwise error {e:.3e} > {tol:.1e}"
    print(f"[state] {label}: normwise {e:.2e} (bound {tol:.0e}); elementwise relative "
          f"{state_err_elementwise(s_gpu, s_ref):.2e} where |S| >= 1e-3 of its head's max", file=sys.stderr)
    return e


def check_bf16_within_ulp(gpu_bits, ref, label=""):
    """Prologue bf16 outputs: within one bf16 ulp of the fp64 value (correct
    rounding is within half an ulp; near-ties may round the other way)."""
    x = oracle.bf16_to_f64(gpu_bits)
    err = np.abs(x - ref)
    bad = err > bf16_ulp(ref)
    assert not bad.any(), f"{label}: {bad.sum()} elements beyond 1 bf16 ulp (worst {err.max():.3e})"
    flips = int(np.count_nonzero(gpu_bits != oracle.round_bf16(ref)))
    return flips


def check_gates(g_gpu, beta_gpu, g_ref, beta_ref, label=""):
    """g: f32 evaluation of exp(-E sp) carries the argument's relative error
    scaled by |ln g| = E sp, so the bound is (8 + 8 |ln g|) u relative, plus
    a few subnormal spacings for g below the normal range.  beta: 8 u."""
    g = g_gpu.astype(np.float64)
    lng = np.abs(np.log(np.maximum(g_ref, 1e-320)))
    tol = (8 + 8 * lng) * U32 * g_ref + 4 * 2.0 ** -149
    bad = np.abs(g - g_ref) > tol
    assert not bad.any(), f"{label}: {bad.sum()} g values out of tolerance"
    b = beta_gpu.astype(np.float64)
    badb = np.abs(b - beta_ref) > 8 * U32 * beta_ref + 2.0 ** -149
    assert not badb.any(), f"{label}: {badb.sum()} beta values out of tolerance"


def layer_uses_chunked(B, T, Hv, Dk, Dv):
    """Whether gdn_layer_core runs the chunked recurrence for these sizes (the
    rule its header states): chunked sizes and T >= 64, or T > 32 with 2048
    state tiles of 16 rows and more, or T > 16 with 4096 and more."""
    if Dk != 128 or Dv % 16 != 0:
        return False
    tiles = B * Hv * (Dv // 16)
    return T >= 64 or (T > 32 and tiles >= 2048) or (T > 16 and tiles >= 4096)


def recurrence_sub(ri, b, hv, rows, Hk, Hv, state=None):
    """Slice the recurrence inputs of one (b, hv) and a subset of its rows
    into a self-contained problem (rows of S evolve independently)."""
    hk = hv // (Hv // Hk)
    f = oracle.bf16_to_f64
    q = f(ri["q"][b:b + 1, :, hk:hk + 1])
    k = f(ri["k"][b:b + 1, :, hk:hk + 1])
    v = f(ri["v"][b:b + 1, :, hv:hv + 1][..., rows])
    g = ri["g"][b:b + 1, :, hv:hv + 1].astype(np.float64)
    be = ri["beta"][b:b + 1, :, hv:hv + 1].astype(np.float64)
    s0 = None if state is None else state[b:b + 1, hv:hv + 1][:, :, rows]
    return q, k, v, g, be, s0


def layer_sub(raw, b, hv, rows, Hk, Hv, Dk, Dv):
    """Slice a layer-core problem to one (b, hv), its k-head's q/k channels
    and a subset of its v channels (the conv is depthwise and the norm is per
    head, so the slice is self-contained)."""
    hk = hv // (Hv // Hk)
    ch = (list(range(hk * Dk, (hk + 1) * Dk))
          + list(range(Hk * Dk + hk * Dk, Hk * Dk + (hk + 1) * Dk))
          + [2 * Hk * Dk + hv * Dv + r for r in rows])
    sl = lambda x: None if x is None else np.ascontiguousarray(x)
    return dict(
        qkv=sl(raw["qkv"][b:b + 1][..., ch]),
        conv_w=sl(raw["conv_w"][ch]),
        conv_state=None if raw["conv_state"] is None else sl(raw["conv_state"][b:b + 1][..., ch]),
        a=sl(raw["a"][b:b + 1, :, hv:hv + 1]),
        b=sl(raw["b"][b:b + 1, :, hv:hv + 1]),
        A_log=sl(raw["A_log"][hv:hv + 1]),
        dt_bias=sl(raw["dt_bias"][hv:hv + 1]),
        state=None if raw["state"] is None else sl(raw["state"][b:b + 1, hv:hv + 1][:, :, rows]),
    )


def guarded(shape, dtype, fill, device=DEV, pad=4096):
    """An output buffer inside canary guard bands: returns (full, view)."""
    n = int(np.prod(shape))
    full = torch.full((n + 2 * pad,), fill, dtype=dtype, device=device)
    return full, full[pad:pad + n].view(shape)


def guards_intact(full, fill, pad=4096):
    head = full[:pad]
    tail = full[-pad:]
    if full.dtype.is_floating_point and math.isnan(fill):
        return bool(torch.isnan(head).all() and torch.isnan(tail).all())
    return bool((head == fill).all() and (tail == fill).all())


def check_epilogue(out_bits, ref, label=""):
    """Output epilogue: every value within one bf16 ulp of the fp64 value (the
    f32 arithmetic is good to about 2^-20 relative, so only values that close
    to a rounding boundary may round the other way: at least 99% of the
    values must carry the bits of the correctly rounded result).  NaN where
    and only where the fp64 value is NaN.  Returns the count of flipped
    roundings."""
    x = oracle.bf16_to_f64(out_bits)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(x), nan_ref), f"{label}: NaN pattern differs"
    err = np.abs(x - ref)[~nan_ref]
    bad = err > bf16_ulp(ref[~nan_ref])
    assert not bad.any(), f"{label}: {bad.sum()} values beyond 1 bf16 ulp (worst {err.max():.3e})"
    flips = int(np.count_nonzero((out_bits != oracle.round_bf16(np.nan_to_num(ref)))[~nan_ref]))
    assert flips <= max(2, 0.01 * out_bits.size), f"{label}: {flips} of {out_bits.size} roundings differ"
    return flips
