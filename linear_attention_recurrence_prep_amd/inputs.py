"""Seeded synthetic inputs for the Gated DeltaNet layer core.

This module is shared by the tests, the benchmark and the smoke check.  It
holds none of the method's arithmetic: it only draws random numbers from fixed
distributions and stores them in the dtypes of the layer's interface
(bf16 as raw ``uint16`` bit patterns, f32 as ``float32``).  Derived inputs
(normalised q/k, the gate g, beta) are computed by whoever consumes the draws.

Every tensor has its own stream:
``numpy.random.Generator(PCG64(SeedSequence([seed, workload_id, tensor_id])))``.

Workloads (shapes and distributions of the pages' own uses: single-sequence
generation, batched decode rows, long prefill):

* ``tiny``       B=1,  T=64,    Hk=2,  Hv=4,  Dk=Dv=32   recurrence inputs
* ``decode_b1``  B=1,  T=1,     Hk=16, Hv=32, Dk=Dv=128  recurrence inputs
* ``decode_b64`` B=64, T=1,     Hk=16, Hv=32, Dk=Dv=128  recurrence inputs
* ``prefill``    B=1,  T=4096,  Hk=16, Hv=32, Dk=Dv=128  mixed qkv, conv K=4,
                                                         zero conv and
                                                         recurrent state
* ``long``       B=4,  T=32768, Hk=16, Hv=32, Dk=Dv=128  mixed qkv, conv K=4,
                                                         zero conv state,
                                                         random recurrent state

Distributions: q, k, v, qkv, a, b ~ N(0, 1); conv weights ~ N(0, 0.1^2);
A_log = log(U[1, 16]); dt_bias ~ N(0, 0.1^2); recurrent state ~ N(0, 0.02^2).
"""
from __future__ import annotations

import math

import numpy as np

SEED = 1234

TENSOR_IDS = {
    "qkv": 0, "conv_w": 1, "conv_state": 2, "a": 3, "b": 4, "A_log": 5,
    "dt_bias": 6, "state": 7, "q_raw": 8, "k_raw": 9, "v": 10,
    "z": 11, "norm_weight": 12, "y": 13, "row_scale": 14, "g_key": 15,
}

WORKLOADS = {
    "tiny": dict(id=0, kind="recurrence", B=1, T=64, Hk=2, Hv=4, Dk=32, Dv=32),
    "decode_b1": dict(id=1, kind="recurrence", B=1, T=1, Hk=16, Hv=32, Dk=128, Dv=128),
    "decode_b64": dict(id=2, kind="recurrence", B=64, T=1, Hk=16, Hv=32, Dk=128, Dv=128),
    "prefill": dict(id=3, kind="layer", B=1, T=4096, Hk=16, Hv=32, Dk=128, Dv=128, K=4,
                    state=False, conv_state=False),
    "long": dict(id=4, kind="layer", B=4, T=32768, Hk=16, Hv=32, Dk=128, Dv=128, K=4,
                 state=True, conv_state=False),
}

_CHUNK = 1 << 22  # draws per generator call for large tensors (fixes the stream)


def generator(workload_id: int, tensor: str, seed: int = SEED) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([seed, int(workload_id), TENSOR_IDS[tensor]])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Store finite float32 draws as bf16 bit patterns (round to nearest even)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) draws stored as bf16 bits; filled in fixed-size chunks so
    tensors of several GiB never need a float64 copy."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[lo:hi] = f32_to_bf16_bits(x)
    return out.reshape(shape)


def normal_f32(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[lo:hi] = x
    return out.reshape(shape)


def a_log_f32(rng: np.random.Generator, Hv: int) -> np.ndarray:
    """A_log = log(U[1, 16]) per v-head, stored f32."""
    return np.log(rng.uniform(1.0, 16.0, size=Hv)).astype(np.float32)


def recurrence_raw(*, B, T, Hk, Hv, Dk, Dv, workload_id=0, state=True, seed=SEED):
    """Raw draws for a recurrence-only call: q_raw, k_raw [B,T,Hk,Dk] and v
    [B,T,Hv,Dv] (bf16 bits, N(0,1)); a, b [B,T,Hv] (bf16 bits, N(0,1));
    A_log, dt_bias [Hv] f32; state [B,Hv,Dv,Dk] f32 N(0, 0.02^2) or None."""
    w = workload_id
    out = dict(
        q_raw=normal_bf16(generator(w, "q_raw", seed), (B, T, Hk, Dk)),
        k_raw=normal_bf16(generator(w, "k_raw", seed), (B, T, Hk, Dk)),
        v=normal_bf16(generator(w, "v", seed), (B, T, Hv, Dv)),
        a=normal_bf16(generator(w, "a", seed), (B, T, Hv)),
        b=normal_bf16(generator(w, "b", seed), (B, T, Hv)),
        A_log=a_log_f32(generator(w, "A_log", seed), Hv),
        dt_bias=normal_f32(generator(w, "dt_bias", seed), (Hv,), 0.1),
        state=normal_f32(generator(w, "state", seed), (B, Hv, Dv, Dk), 0.02) if state else None,
    )
    return out


def layer_raw(*, B, T, Hk, Hv, Dk, Dv, K=4, workload_id=3, state=False, conv_state=False,
              seed=SEED):
    """Raw draws for a layer-core call: qkv [B,T,C] bf16 N(0,1) with
    C = 2*Hk*Dk + Hv*Dv; conv_w [C,K] bf16 N(0, 0.1^2); conv_state
    [B,K-1,C] bf16 N(0,1) or None (zeros); a, b [B,T,Hv] bf16 N(0,1); A_log,
    dt_bias [Hv] f32; state [B,Hv,Dv,Dk] f32 N(0, 0.02^2) or None (zeros)."""
    w = workload_id
    C = 2 * Hk * Dk + Hv * Dv
    return dict(
        qkv=normal_bf16(generator(w, "qkv", seed), (B, T, C)),
        conv_w=normal_bf16(generator(w, "conv_w", seed), (C, K), 0.1),
        conv_state=normal_bf16(generator(w, "conv_state", seed), (B, K - 1, C)) if conv_state else None,
        a=normal_bf16(generator(w, "a", seed), (B, T, Hv)),
        b=normal_bf16(generator(w, "b", seed), (B, T, Hv)),
        A_log=a_log_f32(generator(w, "A_log", seed), Hv),
        dt_bias=normal_f32(generator(w, "dt_bias", seed), (Hv,), 0.1),
        state=normal_f32(generator(w, "state", seed), (B, Hv, Dv, Dk), 0.02) if state else None,
    )


def epilogue_raw(*, B, T, Hv, Dv, workload_id=5, with_y=True, seed=SEED):
    """Raw draws for the output epilogue: z [B,T,Hv,Dv] bf16 N(0,1) (the
    layer's gate projection); norm_weight [Dv] bf16 1 + N(0, 0.1^2); and, for
    a standalone call, y [B,T,Hv,Dv] bf16: N(0,1) rows each scaled by
    2^U[-24, 4], so that some rows are small enough for eps to matter."""
    w = workload_id
    out = dict(
        z=normal_bf16(generator(w, "z", seed), (B, T, Hv, Dv)),
        norm_weight=f32_to_bf16_bits(
            np.float32(1.0) + normal_f32(generator(w, "norm_weight", seed), (Dv,), 0.1)),
    )
    if with_y:
        scale = np.exp2(generator(w, "row_scale", seed).uniform(-24.0, 4.0, (B, T, Hv, 1))).astype(np.float32)
        out["y"] = f32_to_bf16_bits(normal_f32(generator(w, "y", seed), (B, T, Hv, Dv)) * scale)
    return out


def per_key_gate(*, B, T, Hv, Dk, workload_id=6, seed=SEED):
    """A per-key decay gate g [B,T,Hv,Dk] f32 ~ U[0.3, 1)."""
    return generator(workload_id, "g_key", seed).uniform(0.3, 1.0, (B, T, Hv, Dk)).astype(np.float32)


def workload(name: str, seed: int = SEED):
    """Raw draws for a named workload (see the module docstring)."""
    w = WORKLOADS[name]
    dims = {k: w[k] for k in ("B", "T", "Hk", "Hv", "Dk", "Dv")}
    if w["kind"] == "recurrence":
        return recurrence_raw(**dims, workload_id=w["id"], state=True, seed=seed)
    return layer_raw(**dims, K=w["K"], workload_id=w["id"], state=w["state"],
                     conv_state=w["conv_state"], seed=seed)


def scales(Dk: int):
    """Runtime q/k scales of the layer workloads: q is scaled by Dk^-1 and k
    by Dk^-1/2, the inv_scale^2 / inv_scale pair of the op-by-op layer."""
    return 1.0 / Dk, 1.0 / math.sqrt(Dk)
