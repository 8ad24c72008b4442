"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs.  Tolerances (see tests/helpers.py):
  y      within 1 bf16 ulp of the fp64 value + 1e-3 absolute;
  state  per-head normwise max |dS| / max |S| <= 1e-4 (T <= 4096), 1e-3 beyond;
  GQA, batch/head permutation, time split, in-place and NULL-state runs are
  compared bit for bit against the GPU's own reference run.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrence_prep_amd import binding, inputs
from tests import helpers as H

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0   # quiet-NaN bf16 pattern (fits int16)


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.lib()   # raises if the HIP library is not built
    yield
    torch.cuda.synchronize()


def rec_inputs(B, T, Hk, Hv, Dk, Dv, wid, state=True):
    raw = inputs.recurrence_raw(B=B, T=T, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, workload_id=wid, state=state)
    ri = oracle.recurrence_inputs(raw)
    ri["state"] = raw["state"]
    return ri


def gpu_recurrent(ri, state_dev="copy", y_guard=True, mask=None):
    """Run gdn_recurrent(_masked) on device copies of ri; returns (y bits, state f32)."""
    B, T, Hk, Dk = ri["q"].shape
    Hv, Dv = ri["v"].shape[2:]
    d = {k: H.to_dev(ri[k]) for k in ("q", "k", "v", "g", "beta")}
    s_in = H.to_dev(ri["state"]) if ri["state"] is not None else None
    yfull, y = H.guarded((B, T, Hv, Dv), torch.int16, NAN_BF16)
    sfull, s_out = H.guarded((B, Hv, Dv, Dk), torch.float32, float("nan"))
    m = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).to(H.DEV)
    binding.recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], s_in, s_out, y, mask=m)
    torch.cuda.synchronize()
    assert H.guards_intact(yfull, NAN_BF16) and H.guards_intact(sfull, float("nan")), "guard band written"
    return H.bits(y), H.f32(s_out)


def gpu_recurrent_chunked(ri, in_place=False, mask=None):
    """Run gdn_recurrent_chunked on device copies of ri; returns (y bits, state)."""
    B, T, Hk, Dk = ri["q"].shape
    Hv, Dv = ri["v"].shape[2:]
    d = {k: H.to_dev(ri[k]) for k in ("q", "k", "v", "g", "beta")}
    s_in = H.to_dev(ri["state"]) if ri["state"] is not None else None
    yfull, y = H.guarded((B, T, Hv, Dv), torch.int16, NAN_BF16)
    if in_place:
        sfull, s_out = None, s_in
    else:
        sfull, s_out = H.guarded((B, Hv, Dv, Dk), torch.float32, float("nan"))
    nws = binding.recurrent_chunked_workspace_bytes(B, T, Hk, Hv, Dk, Dv)
    wfull, ws = H.guarded((max(nws, 1),), torch.uint8, 0xA5)
    m = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).to(H.DEV)
    binding.recurrent_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], s_in, s_out, y, ws, mask=m)
    torch.cuda.synchronize()
    assert H.guards_intact(yfull, NAN_BF16), "y guard band written"
    assert sfull is None or H.guards_intact(sfull, float("nan")), "state guard band written"
    assert H.guards_intact(wfull, 0xA5), "workspace guard band written"
    return H.bits(y), H.f32(s_out)


def oracle_recurrent(ri):
    f = oracle.bf16_to_f64
    s0 = None if ri["state"] is None else ri["state"].astype(np.float64)
    return oracle.recurrent(f(ri["q"]), f(ri["k"]), f(ri["v"]), ri["g"].astype(np.float64),
                            ri["beta"].astype(np.float64), s0)


# ------------------------------------------------------------ recurrence

REC_CASES = [
    # B, T, Hk, Hv, Dk, Dv, wid           (wid = generator workload id)
    (1, 64, 2, 4, 32, 32, 0),              # tiny workload
    (1, 1, 16, 32, 128, 128, 1),           # decode, B=1
    (64, 1, 16, 32, 128, 128, 2),          # batched decode
    (2, 37, 1, 2, 64, 24, 100),            # ragged T (chunk tail), Dv < rows/block
    (1, 100, 2, 2, 128, 40, 101),          # Dv not a multiple of the block rows
    (1, 19, 1, 1, 256, 8, 102),            # Dk = 256 (32-lane rows)
    (3, 5, 2, 4, 128, 128, 103),           # just above the short-sequence path
    (2, 4, 4, 8, 32, 64, 104),             # short-sequence path, GQA 2
    (1, 70, 1, 4, 64, 64, 105),            # GQA 4, two chunks + tail
    (1, 33, 2, 2, 128, 256, 106),          # Dv = 256, one step past a chunk
]


@pytest.mark.parametrize("case", REC_CASES, ids=lambda c: "B%dT%dHk%dHv%dDk%dDv%d" % c[:6])
def test_recurrent_matches_oracle(case):
    B, T, Hk, Hv, Dk, Dv, wid = case
    say("recurrent", case)
    ri = rec_inputs(B, T, Hk, Hv, Dk, Dv, wid)
    y_bits, s = gpu_recurrent(ri)
    y_ref, s_ref = oracle_recurrent(ri)
    H.check_y(y_bits, y_ref, str(case))
    H.check_state(s, s_ref, 1e-4, str(case))


def test_recurrent_zero_state_and_null_state():
    say("recurrent NULL state")
    ri = rec_inputs(1, 50, 2, 4, 64, 32, 110, state=False)
    y_bits, s = gpu_recurrent(ri)
    y_ref, s_ref = oracle_recurrent(ri)
    H.check_y(y_bits, y_ref)
    H.check_state(s, s_ref, 1e-4)
    ri2 = dict(ri, state=np.zeros((1, 4, 32, 64), np.float32))
    y2, s2 = gpu_recurrent(ri2)
    assert np.array_equal(y_bits, y2) and np.array_equal(s, s2)


def test_recurrent_T0_copies_state():
    say("recurrent T=0")
    ri = rec_inputs(2, 0, 1, 2, 128, 16, 111)
    y_bits, s = gpu_recurrent(ri)
    assert y_bits.size == 0 and np.array_equal(s, ri["state"])
    ri["state"] = None
    _, s = gpu_recurrent(ri)
    assert np.array_equal(s, np.zeros_like(s))


def test_recurrent_in_place_state():
    say("recurrent in place")
    ri = rec_inputs(2, 45, 2, 4, 128, 32, 112)
    y_ref_bits, s_ref = gpu_recurrent(ri)
    d = {k: H.to_dev(ri[k]) for k in ("q", "k", "v", "g", "beta")}
    st = H.to_dev(ri["state"])
    y = torch.empty(2, 45, 4, 32, dtype=torch.int16, device=H.DEV)
    binding.recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], st, st, y)
    torch.cuda.synchronize()
    assert np.array_equal(H.bits(y), y_ref_bits) and np.array_equal(H.f32(st), s_ref)


def test_recurrent_gqa_is_bit_exact_against_repeated_heads():
    say("recurrent GQA")
    ri = rec_inputs(2, 40, 2, 8, 64, 32, 113)
    y1, s1 = gpu_recurrent(ri)
    rep = dict(ri, q=np.repeat(ri["q"], 4, axis=2), k=np.repeat(ri["k"], 4, axis=2))
    y2, s2 = gpu_recurrent(rep)
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)


def test_recurrent_time_split_is_bit_exact():
    say("recurrent T split")
    ri = rec_inputs(1, 90, 1, 2, 128, 32, 114)
    y, s = gpu_recurrent(ri)
    for T1 in (1, 3, 32, 50):
        a = {k: np.ascontiguousarray(ri[k][:, :T1]) for k in ("q", "k", "v", "g", "beta")}
        b = {k: np.ascontiguousarray(ri[k][:, T1:]) for k in ("q", "k", "v", "g", "beta")}
        ya, sa = gpu_recurrent(dict(a, state=ri["state"]))
        yb, sb = gpu_recurrent(dict(b, state=sa))
        assert np.array_equal(np.concatenate([ya, yb], axis=1), y), T1
        assert np.array_equal(sb, s), T1


def test_recurrent_batch_head_permutation_is_bit_exact():
    say("recurrent permutation")
    ri = rec_inputs(3, 20, 2, 4, 64, 16, 115)
    y, s = gpu_recurrent(ri)
    pb, phk, phv = np.array([2, 0, 1]), np.array([1, 0]), np.array([2, 3, 0, 1])
    perm = dict(q=ri["q"][pb][:, :, phk], k=ri["k"][pb][:, :, phk], v=ri["v"][pb][:, :, phv],
                g=ri["g"][pb][:, :, phv], beta=ri["beta"][pb][:, :, phv], state=ri["state"][pb][:, phv])
    y2, s2 = gpu_recurrent({k: np.ascontiguousarray(v) for k, v in perm.items()})
    assert np.array_equal(y2, y[pb][:, :, phv]) and np.array_equal(s2, s[pb][:, phv])


def test_recurrent_repeat_runs_are_bitwise_identical():
    say("recurrent determinism")
    ri = rec_inputs(4, 77, 2, 4, 128, 64, 116)
    y1, s1 = gpu_recurrent(ri)
    y2, s2 = gpu_recurrent(ri)
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)


def test_recurrent_invariants_on_gpu():
    # beta = 0, g = 1: the state is carried unchanged (exactly)
    say("recurrent invariants")
    ri = rec_inputs(1, 10, 1, 2, 64, 16, 117)
    ri["g"][:] = 1.0
    ri["beta"][:] = 0.0
    _, s = gpu_recurrent(ri)
    assert np.array_equal(s, ri["state"])
    # g = 0 at the last step: S = beta v k^T regardless of the history
    ri = rec_inputs(1, 10, 1, 2, 64, 16, 118)
    ri["g"][:, -1] = 0.0
    _, s = gpu_recurrent(ri)
    f = oracle.bf16_to_f64
    for h in range(2):
        ref = np.outer(f(ri["v"][0, -1, h]) * ri["beta"][0, -1, h], f(ri["k"][0, -1, 0]))
        np.testing.assert_allclose(s[0, h], ref, rtol=2 ** -22, atol=0)


# --------------------------------------------------------------- prologue

def layer_inputs(B, T, Hk, Hv, Dk, Dv, K, wid, state=True, conv_state=True):
    return inputs.layer_raw(B=B, T=T, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, K=K, workload_id=wid,
                            state=state, conv_state=conv_state)


def gpu_prep(raw, Hk, Hv, Dk, Dv, qs, ks, eps=1e-6, in_place=False, write_cs=True):
    B, T, C = raw["qkv"].shape
    K = raw["conv_w"].shape[1]
    d = {k: H.to_dev(raw[k]) for k in ("qkv", "conv_w", "conv_state", "a", "b", "A_log", "dt_bias")}
    q = torch.empty(B, T, Hk, Dk, dtype=torch.int16, device=H.DEV)
    k = torch.empty_like(q)
    v = torch.empty(B, T, Hv, Dv, dtype=torch.int16, device=H.DEV)
    g = torch.empty(B, T, Hv, dtype=torch.float32, device=H.DEV)
    beta = torch.empty_like(g)
    if in_place:
        cs_out = d["conv_state"]
    else:
        cs_out = torch.full((B, K - 1, C), NAN_BF16, dtype=torch.int16, device=H.DEV) if write_cs else None
    binding.prep(d["qkv"], d["conv_w"], d["conv_state"], cs_out, d["a"], d["b"], d["A_log"],
                 d["dt_bias"], q, k, v, g, beta, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, q_scale=qs,
                 k_scale=ks, eps=eps)
    torch.cuda.synchronize()
    return dict(q=H.bits(q), k=H.bits(k), v=H.bits(v), g=H.f32(g), beta=H.f32(beta),
                conv_state=None if cs_out is None else H.bits(cs_out))


PREP_CASES = [
    # B, T, Hk, Hv, Dk, Dv, K, conv_state, wid
    (1, 64, 2, 4, 32, 32, 4, False, 200),
    (2, 37, 2, 4, 64, 24, 4, True, 201),
    (1, 50, 4, 8, 128, 128, 3, True, 202),
    (3, 17, 1, 2, 256, 48, 2, True, 203),
    (2, 2, 16, 32, 128, 128, 4, True, 204),      # T < K - 1
    (1, 300, 16, 32, 128, 128, 4, False, 205),   # full-width channels, several token chunks
]


@pytest.mark.parametrize("case", PREP_CASES, ids=lambda c: "B%dT%dHk%dHv%dDk%dDv%dK%d" % c[:7])
def test_prep_matches_oracle(case):
    B, T, Hk, Hv, Dk, Dv, K, cs, wid = case
    say("prep", case)
    raw = layer_inputs(B, T, Hk, Hv, Dk, Dv, K, wid, conv_state=cs)
    qs, ks = 1.0 / Dk, Dk ** -0.5
    out = gpu_prep(raw, Hk, Hv, Dk, Dv, qs, ks)
    ref = oracle.prep(raw["qkv"], raw["conv_w"], raw["conv_state"], raw["a"], raw["b"], raw["A_log"],
                      raw["dt_bias"], Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, q_scale=qs, k_scale=ks)
    flips = sum(H.check_bf16_within_ulp(out[n], ref[n], n) for n in ("q", "k", "v"))
    n_el = out["q"].size * 2 + out["v"].size
    assert flips <= max(4, n_el // 1000), f"{flips} of {n_el} roundings differ from nearest-even"
    H.check_gates(out["g"], out["beta"], ref["g"], ref["beta"])
    assert np.array_equal(out["conv_state"], ref["conv_state"])


def test_prep_extreme_activations_and_gates():
    """Conv outputs deep in SiLU's negative tail (where e^-u overflows f32 and
    the true value is a tiny normal or subnormal number) and gate inputs far
    out on both sides, against the oracle."""
    B, T, Hk, Hv, Dk, Dv, K = 1, 24, 1, 2, 32, 32, 4
    say("prep extremes")
    raw = layer_inputs(B, T, Hk, Hv, Dk, Dv, K, 215)
    f = oracle.bf16_to_f64
    tail = np.array([-87.0, -88.0, -89.0, -92.0, -95.0, -100.0, -103.0, -110.0, -200.0, -1e4, 88.0, 100.0,
                     -20.0, 20.0, 0.0, -0.0, -87.5, -96.0, -101.0, -104.0, -3.0, 3.0, -88.5, -150.0])
    cw = f(raw["conv_w"])
    x = f(raw["qkv"])
    for c in (5, Dk + 7, 2 * Dk + 3, 2 * Dk + Dv + 11):    # a q, a k and two v channels
        cw[c] = [0.0, 0.0, 0.0, 1.0]                          # the newest tap only: u = x
        x[0, :, c] = tail
    raw["conv_w"], raw["qkv"] = oracle.round_bf16(cw), oracle.round_bf16(x)
    raw["b"] = oracle.round_bf16(np.resize(tail, (B, T, Hv)) * np.array([1.0, -1.0]))
    raw["a"] = oracle.round_bf16(np.resize(tail[::-1], (B, T, Hv)))
    qs, ks = 1.0 / Dk, Dk ** -0.5
    out = gpu_prep(raw, Hk, Hv, Dk, Dv, qs, ks)
    ref = oracle.prep(raw["qkv"], raw["conv_w"], raw["conv_state"], raw["a"], raw["b"], raw["A_log"],
                      raw["dt_bias"], Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, q_scale=qs, k_scale=ks)
    for n in ("q", "k", "v"):
        H.check_bf16_within_ulp(out[n], ref[n], n)
    H.check_gates(out["g"], out["beta"], ref["g"], ref["beta"])
    assert oracle.bf16_to_f64(out["v"][0, 2, 0, 3]) < 0     # silu(-89) is a normal bf16 number


def test_prep_conv_state_in_place_and_T0():
    say("prep in-place conv state / T=0")
    raw = layer_inputs(2, 9, 2, 4, 64, 16, 4, 210)
    ref = gpu_prep(raw, 2, 4, 64, 16, 0.1, 0.2)
    ip = gpu_prep(raw, 2, 4, 64, 16, 0.1, 0.2, in_place=True)
    for n in ("q", "k", "v", "g", "beta", "conv_state"):
        assert np.array_equal(ip[n], ref[n]), n
    raw0 = layer_inputs(2, 0, 2, 4, 64, 16, 4, 211)
    out0 = gpu_prep(raw0, 2, 4, 64, 16, 0.1, 0.2)
    assert np.array_equal(out0["conv_state"], raw0["conv_state"])
    raw0["conv_state"] = None
    out0 = gpu_prep(raw0, 2, 4, 64, 16, 0.1, 0.2)
    assert not out0["conv_state"].any()


# ------------------------------------------------------------- layer core

def gpu_layer_core(raw, Hk, Hv, Dk, Dv, qs, ks, eps=1e-6, mask=None, cs_in_place=False):
    B, T, C = raw["qkv"].shape
    K = raw["conv_w"].shape[1]
    d = {k: H.to_dev(raw[k]) for k in ("qkv", "conv_w", "conv_state", "a", "b", "A_log", "dt_bias",
                                       "state")}
    y = torch.empty(B, T, Hv, Dv, dtype=torch.int16, device=H.DEV)
    s_out = torch.empty(B, Hv, Dv, Dk, dtype=torch.float32, device=H.DEV)
    cs_out = d["conv_state"] if cs_in_place else torch.empty(B, K - 1, C, dtype=torch.int16, device=H.DEV)
    nws = binding.layer_core_workspace_bytes(B, T, Hk, Hv, Dk, Dv)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=H.DEV)
    m = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).to(H.DEV)
    binding.layer_core(d["qkv"], d["conv_w"], d["conv_state"], cs_out, d["a"], d["b"], d["A_log"],
                       d["dt_bias"], d["state"], s_out, y, ws, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv,
                       q_scale=qs, k_scale=ks, eps=eps, mask=m)
    torch.cuda.synchronize()
    return H.bits(y), H.f32(s_out), H.bits(cs_out)


def oracle_on_gpu_prologue(p, state, mask=None):
    """The oracle's recurrence on the prologue outputs the device produced
    (stored bf16 q, k, v and f32 g, beta from gdn_prep): the end-to-end
    reference that keeps the prologue's rare near-tie roundings, which the
    prologue tests bound separately, out of the recurrence's error."""
    f = oracle.bf16_to_f64
    s0 = None if state is None else state.astype(np.float64)
    return oracle.recurrent(f(p["q"]), f(p["k"]), f(p["v"]), p["g"].astype(np.float64),
                            p["beta"].astype(np.float64), s0, mask=mask)


def state_tol_for(T):
    """The state bound: 1e-4 per head, normwise, up to T = 4096; 1e-3 beyond."""
    return 1e-4 if T <= 4096 else 1e-3


def compare_core(label, y, s, y_r, s_r, y_o, s_o, tol):
    """y (bits) and state s of a layer-core run against the oracle's
    recurrence on the device's prologue outputs (y_r, s_r): y to the strict
    bounds, state within tol.  Against the oracle's own prologue (y_o, s_o):
    y within 1 ulp + 1e-3, state within tol plus the effect, measured in
    fp64, of the prologue outputs the device rounded to the other bf16
    neighbour (the distance between the two references)."""
    fy = H.check_y(y, y_r, label)
    e = H.check_state(s, s_r, tol, label)
    H.check_y(y, y_o, label + " (oracle prologue)", strict=False)
    e_flip = H.state_err(s_r, s_o)
    e_o = H.state_err(s, s_o)
    assert e_o <= tol * (1 + e_flip) + e_flip, f"{label}: state {e_o:.3e} from the oracle's own prologue"
    say(label, f"state err {e:.2e} (vs the oracle prologue {e_o:.2e}; prologue roundings alone {e_flip:.2e});",
        "y", {k: f"{v:.3g}" for k, v in fy.items()})
    return e


def check_core(label, y, s, p, raw, Hk, Hv, Dk, Dv, qs, ks, mask=None, tol=1e-4):
    """A whole layer-core run (compare_core) whose prologue outputs from
    gdn_prep are p; returns the oracle's conv-state tail."""
    y_r, s_r = oracle_on_gpu_prologue(p, raw["state"], mask)
    y_o, s_o, cs_o = oracle.layer_core(raw["qkv"], raw["conv_w"], raw["conv_state"], raw["a"], raw["b"],
                                       raw["A_log"], raw["dt_bias"], raw["state"], Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv,
                                       q_scale=qs, k_scale=ks, mask=mask)
    compare_core(label, y, s, y_r, s_r, y_o, s_o, tol)
    return cs_o


def check_core_heads(label, y, s, p, raw, heads, rows, Hk, Hv, Dk, Dv, qs, ks, tol):
    """compare_core on sampled (b, hv) heads and rows of a large run, each
    recomputed by the oracle as a self-contained sub-problem: the recurrence
    on the device's prologue outputs, and the whole layer core from the
    head's own channels."""
    ri = dict(q=p["q"], k=p["k"], v=p["v"], g=p["g"], beta=p["beta"])
    worst = 0.0
    for b, hv in heads:
        lab = f"{label} b={b} hv={hv}"
        y_r, s_r = oracle.recurrent(*H.recurrence_sub(ri, b, hv, rows, Hk, Hv, raw["state"]))
        sub = H.layer_sub(raw, b, hv, rows, Hk, Hv, Dk, Dv)
        y_o, s_o, _ = oracle.layer_core(sub["qkv"], sub["conv_w"], sub["conv_state"], sub["a"], sub["b"],
                                        sub["A_log"], sub["dt_bias"], sub["state"], Hk=1, Hv=1, Dk=Dk,
                                        Dv=len(rows), q_scale=qs, k_scale=ks)
        yh = np.ascontiguousarray(y[b:b + 1, :, hv:hv + 1][..., rows])
        sh = s[b:b + 1, hv:hv + 1][:, :, rows]
        worst = max(worst, compare_core(lab, yh, sh, y_r, s_r, y_o, s_o, tol))
    return worst


CORE_CASES = [
    # B, T, Hk, Hv, Dk, Dv, K, wid
    (1, 64, 2, 4, 32, 32, 4, 300),
    (2, 45, 2, 4, 64, 24, 3, 301),
    (1, 130, 4, 8, 128, 128, 4, 302),
    (1, 100, 3, 3, 128, 64, 2, 303),       # GQA 1: one v-head per preparation block, conv K=2
    (1, 70, 2, 4, 128, 96, 3, 305),        # two v-heads per preparation block, Dv < 128, K=3
]


@pytest.mark.parametrize("case", CORE_CASES, ids=lambda c: "B%dT%dHk%dHv%dDk%dDv%dK%d" % c[:7])
def test_layer_core_matches_oracle(case):
    B, T, Hk, Hv, Dk, Dv, K, wid = case
    say("layer_core", case)
    raw = layer_inputs(B, T, Hk, Hv, Dk, Dv, K, wid)
    qs, ks = 1.0 / Dk, Dk ** -0.5
    y, s, cs = gpu_layer_core(raw, Hk, Hv, Dk, Dv, qs, ks)
    p = gpu_prep(raw, Hk, Hv, Dk, Dv, qs, ks)
    cs_ref = check_core(str(case), y, s, p, raw, Hk, Hv, Dk, Dv, qs, ks)
    assert np.array_equal(cs, cs_ref)


@pytest.mark.parametrize("shape", [(2, 70, 2, 4, 128, 64, 4), (2, 40, 2, 4, 128, 64, 4), (1, 90, 1, 2, 64, 32, 4),
                                   (1, 100, 3, 3, 128, 64, 2), (2, 96, 2, 6, 128, 32, 3),
                                   (1, 70, 2, 4, 128, 96, 3), (2, 96, 1, 4, 128, 32, 4),
                                   (1, 80, 1, 2, 128, 256, 4), (16, 24, 4, 32, 128, 128, 4),
                                   (8, 40, 4, 32, 128, 128, 4), (8, 32, 4, 32, 128, 128, 4)],
                         ids=["chunked", "short", "Dk64", "chunked_G1_K2", "chunked_G3_K3", "chunked_G2_Dv96_K3",
                              "chunked_G4", "chunked_Dv256_unfused", "short_wide_chunked", "mid_wide_chunked",
                              "short_wide_per_step"])
def test_layer_core_equals_prep_then_recurrent(shape):
    """The layer core is the prologue followed by the chunked recurrence
    (the rule of tests.helpers.layer_uses_chunked) or else the per-step one, bit for bit
    (in the chunked form the prologue runs inside the chunk preparation, one
    or two v-heads per block by the parity of the GQA group size)."""
    B, T, Hk, Hv, Dk, Dv, K = shape
    say("layer_core composition", shape)
    raw = layer_inputs(B, T, Hk, Hv, Dk, Dv, K, 310)
    y, s, cs = gpu_layer_core(raw, Hk, Hv, Dk, Dv, 0.01, 0.09)
    p = gpu_prep(raw, Hk, Hv, Dk, Dv, 0.01, 0.09)
    ri = dict(q=p["q"], k=p["k"], v=p["v"], g=p["g"], beta=p["beta"], state=raw["state"])
    chunked = H.layer_uses_chunked(B, T, Hv, Dk, Dv)
    y2, s2 = gpu_recurrent_chunked(ri) if chunked else gpu_recurrent(ri)
    assert np.array_equal(y, y2) and np.array_equal(s, s2) and np.array_equal(cs, p["conv_state"])


@pytest.mark.parametrize("shape", [(2, 96, 2, 4, 128, 64, 4), (1, 70, 2, 2, 128, 128, 3), (2, 96, 1, 4, 128, 32, 4),
                                   (2, 5, 2, 4, 128, 64, 4), (1, 2, 2, 4, 128, 32, 4)],
                         ids=["chunked_G2_fused", "chunked_G1_fused", "chunked_G4_fused_tail_copy", "per_step",
                              "T_below_K"])
def test_layer_core_conv_state_in_place(shape):
    """The conv state updated in place (conv_state_out == conv_state_in) gives
    the same bits as a separate output, in the chunked form with the prologue
    fused (one preparation block per k-head writes the conv state; with more,
    a copy after the preparation does) and in the per-step form."""
    B, T, Hk, Hv, Dk, Dv, K = shape
    say("layer_core conv state in place", shape)
    raw = layer_inputs(B, T, Hk, Hv, Dk, Dv, K, 320)
    y, s, cs = gpu_layer_core(raw, Hk, Hv, Dk, Dv, 0.01, 0.09)
    y2, s2, cs2 = gpu_layer_core(raw, Hk, Hv, Dk, Dv, 0.01, 0.09, cs_in_place=True)
    assert np.array_equal(y, y2) and np.array_equal(s, s2) and np.array_equal(cs, cs2)


DECODE_CASES = [
    # B, Hk, Hv, Dk, Dv, K, masked, conv state in place, wid
    (64, 16, 32, 128, 128, 4, False, True, 330),      # the batched-decode workload
    (128, 2, 4, 64, 32, 3, True, False, 331),
    (256, 1, 4, 256, 48, 2, True, True, 332),         # four v-heads per k-head, Dv not a multiple of 32
    (32, 8, 8, 32, 16, 4, False, False, 333),         # one v-head per k-head
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "B%dHk%dHv%dDk%dDv%dK%d-m%dip%d" % c[:8])
def test_layer_core_single_token_decode(case):
    """Single-token decode of a large batch (one launch: prologue and step per
    (b, k-head) block) equals the prologue followed by the per-step
    recurrence bit for bit, with masks and the conv state in place, and the
    oracle within the tolerances."""
    B, Hk, Hv, Dk, Dv, K, masked, ip, wid = case
    say("layer_core decode", case)
    raw = layer_inputs(B, 1, Hk, Hv, Dk, Dv, K, wid)
    qs, ks = 1.0 / Dk, Dk ** -0.5
    mask = step_mask(wid, B, 1, p=0.6) if masked else None
    y, s, cs = gpu_layer_core(raw, Hk, Hv, Dk, Dv, qs, ks, mask=mask, cs_in_place=ip)
    p = gpu_prep(raw, Hk, Hv, Dk, Dv, qs, ks)
    ri = dict(q=p["q"], k=p["k"], v=p["v"], g=p["g"], beta=p["beta"], state=raw["state"])
    y2, s2 = gpu_recurrent(ri, mask=mask)
    assert np.array_equal(y, y2) and np.array_equal(s, s2) and np.array_equal(cs, p["conv_state"])
    cs_ref = check_core(str(case), y, s, p, raw, Hk, Hv, Dk, Dv, qs, ks, mask=mask)
    assert np.array_equal(cs, cs_ref)


@pytest.mark.parametrize("q_scale", ["mlex", "rms_x_dk_half"])
def test_prefill_workload_full_size_sampled(q_scale):
    """The T=4096 prefill workload at full size through the layer core (the
    headline step: prologue fused into the chunk preparation); four whole
    v-heads against the oracle's recurrence on the device's own prologue
    outputs (state 1e-4, strict y bounds) and against the oracle's own
    prologue.  Both readings of the q scale: Dk^-1 (the mlex page scales q
    by inv_scale squared) and Dk^-1/2 (RMS-normalised x Dk^-1/2 as the
    workload's description states for q and k)."""
    say("prefill workload full size", q_scale)
    w = inputs.WORKLOADS["prefill"]
    Hk, Hv, Dk, Dv = w["Hk"], w["Hv"], w["Dk"], w["Dv"]
    raw = inputs.workload("prefill")
    qs, ks = inputs.scales(Dk)
    if q_scale == "rms_x_dk_half":
        qs = Dk ** -0.5
    y, s, cs = gpu_layer_core(raw, Hk, Hv, Dk, Dv, qs, ks)
    assert not np.isnan(s).any()
    p = gpu_prep(raw, Hk, Hv, Dk, Dv, qs, ks)
    heads = [(0, hv) for hv in (0, 5, 17, 31)]
    worst = check_core_heads("prefill " + q_scale, y, s, p, raw, heads, list(range(Dv)), Hk, Hv, Dk, Dv, qs, ks,
                             1e-4)
    say("prefill state normwise err", worst)
    assert np.array_equal(cs, raw["qkv"][:, -(w["K"] - 1):])


@pytest.mark.parametrize("workload", ["prefill", "long"])
def test_layer_core_equals_composition_full_size(workload):
    """At the prefill workload's full grid, and for one whole sequence of the
    long workload (T = 32768), the layer core (prologue fused into the chunk
    preparation) is bit for bit gdn_prep followed by gdn_recurrent_chunked."""
    say("layer core composition full size", workload)
    w = inputs.WORKLOADS[workload]
    Hk, Hv, Dk, Dv = w["Hk"], w["Hv"], w["Dk"], w["Dv"]
    raw = inputs.workload(workload)
    if workload == "long":
        b = 2
        raw = {k: (None if v is None else np.ascontiguousarray(v[b:b + 1]) if k in
                   ("qkv", "conv_state", "a", "b", "state") else v) for k, v in raw.items()}
    qs, ks = inputs.scales(Dk)
    B, T = raw["qkv"].shape[:2]
    assert H.layer_uses_chunked(B, T, Hv, Dk, Dv)
    y, s, cs = gpu_layer_core(raw, Hk, Hv, Dk, Dv, qs, ks)
    p = gpu_prep(raw, Hk, Hv, Dk, Dv, qs, ks)
    ri = dict(q=p["q"], k=p["k"], v=p["v"], g=p["g"], beta=p["beta"], state=raw["state"])
    y2, s2 = gpu_recurrent_chunked(ri)
    assert np.array_equal(cs, p["conv_state"])
    assert np.array_equal(s, s2), "state differs from the composition"
    assert np.array_equal(y, y2), "y differs from the composition"


def test_prefill_workload_recurrence_strict():
    """Recurrence at the prefill workload's size on oracle-prepared inputs
    (the oracle's own prologue, rounded to the stored dtypes), sampled heads,
    strict 1e-4 state bound."""
    say("prefill recurrence strict")
    w = inputs.WORKLOADS["prefill"]
    Hk, Hv, Dk, Dv, T = w["Hk"], w["Hv"], w["Dk"], w["Dv"], w["T"]
    raw = inputs.workload("prefill")
    qs, ks = inputs.scales(Dk)
    p = oracle.prep(raw["qkv"], raw["conv_w"], raw["conv_state"], raw["a"], raw["b"], raw["A_log"],
                    raw["dt_bias"], Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, q_scale=qs, k_scale=ks)
    ri = dict(q=oracle.round_bf16(p["q"]), k=oracle.round_bf16(p["k"]), v=oracle.round_bf16(p["v"]),
              g=oracle.round_f32(p["g"]), beta=oracle.round_f32(p["beta"]), state=None)
    y, s = gpu_recurrent(ri)
    for hv in (1, 12, 30):
        args = H.recurrence_sub(ri, 0, hv, list(range(Dv)), Hk, Hv)
        y_ref, s_ref = oracle.recurrent(*args)
        H.check_y(y[:, :, hv:hv + 1], y_ref, f"hv={hv}")
        H.check_state(s[:, hv:hv + 1], s_ref, 1e-4, f"hv={hv}")


def test_prefill_workload_chunked_recurrence_strict():
    """The chunked recurrence at the prefill workload's full size (the form the
    layer core runs there), on oracle-prepared inputs: sampled heads, all
    rows, strict 1e-4 state bound."""
    say("prefill chunked recurrence strict")
    w = inputs.WORKLOADS["prefill"]
    Hk, Hv, Dk, Dv = w["Hk"], w["Hv"], w["Dk"], w["Dv"]
    raw = inputs.workload("prefill")
    qs, ks = inputs.scales(Dk)
    p = oracle.prep(raw["qkv"], raw["conv_w"], raw["conv_state"], raw["a"], raw["b"], raw["A_log"],
                    raw["dt_bias"], Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, q_scale=qs, k_scale=ks)
    ri = dict(q=oracle.round_bf16(p["q"]), k=oracle.round_bf16(p["k"]), v=oracle.round_bf16(p["v"]),
              g=oracle.round_f32(p["g"]), beta=oracle.round_f32(p["beta"]), state=None)
    y, s = gpu_recurrent_chunked(ri)
    worst = 0.0
    for hv in (2, 15, 29):
        args = H.recurrence_sub(ri, 0, hv, list(range(Dv)), Hk, Hv)
        y_ref, s_ref = oracle.recurrent(*args)
        H.check_y(y[:, :, hv:hv + 1], y_ref, f"hv={hv}")
        worst = max(worst, H.check_state(s[:, hv:hv + 1], s_ref, 1e-4, f"hv={hv}"))
    say("prefill chunked state normwise err", worst)


@pytest.mark.parametrize("q_scale", ["mlex", "rms_x_dk_half"])
def test_long_workload_full_size_sampled(q_scale):
    """B=4, T=32768 with random initial state: the full layer core on the GPU;
    8 rows of 3 (b, hv) heads over the whole sequence against the oracle's
    recurrence on the device's own prologue outputs (long-horizon drift:
    state 1e-3, strict y bounds) and against the oracle's own prologue.  Both
    readings of the q scale, as at the prefill workload."""
    say("long workload full size", q_scale)
    w = inputs.WORKLOADS["long"]
    Hk, Hv, Dk, Dv, T = w["Hk"], w["Hv"], w["Dk"], w["Dv"], w["T"]
    raw = inputs.workload("long")
    qs, ks = inputs.scales(Dk)
    if q_scale == "rms_x_dk_half":
        qs = Dk ** -0.5
    y, s, cs = gpu_layer_core(raw, Hk, Hv, Dk, Dv, qs, ks)
    assert not np.isnan(s).any()
    p = gpu_prep(raw, Hk, Hv, Dk, Dv, qs, ks)
    rows = [0, 9, 31, 64, 77, 100, 126, 127]
    worst = check_core_heads("long " + q_scale, y, s, p, raw, ((0, 0), (1, 13), (3, 31)), rows, Hk, Hv, Dk, Dv,
                             qs, ks, state_tol_for(T))
    say("long state normwise err", worst)


@pytest.mark.parametrize("T", [1, 8, 40], ids=["step_kernel", "chunk_kernel", "chunk_kernel_2chunks"])
def test_y_bf16_rounding_ties_to_even(T):
    """y = S q is rounded to bf16 on the device.  With a zero state, k = q = e_0
    and g = 0 every step, y_t = v * beta_t exactly in f32 (powers of two times
    beta), so the bf16 code is decided by the rounding alone; it must be the
    nearest-even rounding of that exact value."""
    say("y rounding ties", T)
    Dk, Dv = 32, 8
    one = 0x3F80
    q = np.zeros((1, T, 1, Dk), np.uint16)
    q[..., 0] = one
    k = q.copy()
    vals = np.array([1.0, -1.0, 2.0, 0.5, 4.0, -0.25, 1.0, -8.0])
    v = np.tile(oracle.round_bf16(vals), (1, T, 1, 1)).reshape(1, T, 1, Dv)
    betas = np.array([1 + 2 ** -8, 1 + 2 ** -7 + 2 ** -8, 1 + 2 ** -8 + 2 ** -20, 1 - 2 ** -9,
                      1 + 3 * 2 ** -8, 0.5 + 2 ** -10, 1.0, 1 - 3 * 2 ** -10], np.float64)
    beta = np.resize(betas, T).astype(np.float32).reshape(1, T, 1)
    g = np.zeros((1, T, 1), np.float32)
    y_bits, _ = gpu_recurrent(dict(q=q, k=k, v=v, g=g, beta=beta, state=None))
    exact = vals[None, :] * beta.reshape(T, 1).astype(np.float64)    # exact in f32 and f64
    assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)
    expect = oracle.round_bf16(exact)
    assert np.array_equal(y_bits.reshape(T, Dv), expect)


# ------------------------------------------------- chunked (matrix-core) form

CHUNK_CASES = [
    # B, T, Hk, Hv, Dk, Dv, wid
    (1, 64, 2, 4, 128, 32, 400),           # two whole chunks
    (2, 33, 1, 2, 128, 16, 401),           # one step past a chunk
    (1, 100, 2, 2, 128, 48, 402),          # ragged tail
    (3, 5, 2, 4, 128, 128, 403),           # shorter than a chunk
    (64, 1, 16, 32, 128, 128, 2),          # decode-sized batch, one step
    (1, 257, 4, 8, 128, 64, 404),          # GQA 2, nine chunks
    (1, 70, 2, 4, 128, 256, 405),          # Dv = 256: two v slices, two heads per preparation block
    (2, 50, 3, 3, 128, 160, 406),          # Dv = 160 (128 + 32), one head per preparation block
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=lambda c: "B%dT%dHk%dHv%dDk%dDv%d" % c[:6])
def test_recurrent_chunked_matches_oracle(case):
    B, T, Hk, Hv, Dk, Dv, wid = case
    say("recurrent_chunked", case)
    ri = rec_inputs(B, T, Hk, Hv, Dk, Dv, wid)
    y_bits, s = gpu_recurrent_chunked(ri)
    y_ref, s_ref = oracle_recurrent(ri)
    H.check_y(y_bits, y_ref, str(case))
    e = H.check_state(s, s_ref, 1e-4, str(case))
    say("chunked state err", e)


@pytest.mark.parametrize("B,Hv,Dv,zero_state", [(2, 32, 128, False), (3, 32, 64, False), (3, 32, 128, False),
                                                  (5, 32, 64, False), (4, 32, 128, True), (2, 32, 192, False)],
                         ids=["two_tiles_B2", "two_tiles_B3_Dv64", "wave_pairs_B3", "wave_pairs_B5_Dv64",
                              "wave_pairs_B4_zero_state", "wave_pairs_B2_Dv192"])
def test_recurrent_chunked_two_row_tiles(B, Hv, Dv, zero_state):
    """Once B*Hv*Dv/16 exceeds the CU count the sequential pass serves two
    16-row tiles per block, and once it exceeds twice the CU count two waves
    per tile, one per half of the key columns, four tiles per block
    (chunk_seq_pairs_kernel); one tile per block below that.  Sequences of a
    batch are independent, so each must be bit-identical to itself run alone
    (a smaller grid: one or two tiles per block), and the batch must meet
    the oracle.  T = 100 ends in a partial chunk; the last sequence has
    masked steps."""
    say("recurrent_chunked two row tiles / wave pairs", B, Hv, Dv, zero_state)
    ri = rec_inputs(B, 100, Hv // 2, Hv, 128, Dv, 421)
    if zero_state:
        ri["state"] = None
    mask = np.ones((B, 100), dtype=np.uint8)
    mask[-1, 37:41] = 0
    y, s = gpu_recurrent_chunked(ri, mask=mask)
    for b in range(B):
        one = {k: (None if ri[k] is None else np.ascontiguousarray(ri[k][b:b + 1]))
               for k in ("q", "k", "v", "g", "beta", "state")}
        y1, s1 = gpu_recurrent_chunked(one, mask=mask[b:b + 1])
        assert np.array_equal(y[b:b + 1], y1) and np.array_equal(s[b:b + 1], s1), b
    st = np.zeros(s.shape) if ri["state"] is None else ri["state"].astype(np.float64)
    y_ref, s_ref = oracle.recurrent(*[oracle.bf16_to_f64(ri[k]) for k in ("q", "k", "v")],
                                    ri["g"].astype(np.float64), ri["beta"].astype(np.float64), st, mask=mask)
    H.check_y(y, y_ref, "two tiles / wave pairs")
    H.check_state(s, s_ref, 1e-4, "two tiles / wave pairs")


def test_recurrent_chunked_properties():
    say("recurrent_chunked properties")
    ri = rec_inputs(2, 96, 2, 8, 128, 32, 410)
    y, s = gpu_recurrent_chunked(ri)
    # repeat run: bitwise identical
    y2, s2 = gpu_recurrent_chunked(ri)
    assert np.array_equal(y, y2) and np.array_equal(s, s2)
    # GQA against explicitly repeated k-heads: bitwise identical
    rep = dict(ri, q=np.repeat(ri["q"], 4, axis=2), k=np.repeat(ri["k"], 4, axis=2))
    y3, s3 = gpu_recurrent_chunked(rep)
    assert np.array_equal(y, y3) and np.array_equal(s, s3)
    # in place
    y4, s4 = gpu_recurrent_chunked(ri, in_place=True)
    assert np.array_equal(y, y4) and np.array_equal(s, s4)
    # split at a chunk boundary, state carried: bitwise identical
    for T1 in (32, 64):
        a = {k: np.ascontiguousarray(ri[k][:, :T1]) for k in ("q", "k", "v", "g", "beta")}
        b = {k: np.ascontiguousarray(ri[k][:, T1:]) for k in ("q", "k", "v", "g", "beta")}
        ya, sa = gpu_recurrent_chunked(dict(a, state=ri["state"]))
        yb, sb = gpu_recurrent_chunked(dict(b, state=sa))
        assert np.array_equal(np.concatenate([ya, yb], axis=1), y), T1
        assert np.array_equal(sb, s), T1
    # NULL state equals an explicit zero state
    z = dict(ri, state=None)
    y5, s5 = gpu_recurrent_chunked(z)
    y6, s6 = gpu_recurrent_chunked(dict(ri, state=np.zeros_like(ri["state"])))
    assert np.array_equal(y5, y6) and np.array_equal(s5, s6)
    # T = 0 copies the state
    e = {k: np.ascontiguousarray(ri[k][:, :0]) for k in ("q", "k", "v", "g", "beta")}
    _, s7 = gpu_recurrent_chunked(dict(e, state=ri["state"]))
    assert np.array_equal(s7, ri["state"])


def test_recurrent_chunked_invariants():
    say("recurrent_chunked invariants")
    # beta = 0, g = 1: the state is carried unchanged
    ri = rec_inputs(1, 40, 1, 2, 128, 16, 411)
    ri["g"][:] = 1.0
    ri["beta"][:] = 0.0
    _, s = gpu_recurrent_chunked(ri)
    np.testing.assert_allclose(s, ri["state"], rtol=0, atol=0)
    # g = 0 at the last step: S = beta v k^T regardless of the history
    ri = rec_inputs(1, 40, 1, 2, 128, 16, 412)
    ri["g"][:, -1] = 0.0
    _, s = gpu_recurrent_chunked(ri)
    f = oracle.bf16_to_f64
    for h in range(2):
        ref = np.outer(f(ri["v"][0, -1, h]) * ri["beta"][0, -1, h], f(ri["k"][0, -1, 0]))
        np.testing.assert_allclose(s[0, h], ref, rtol=1e-6, atol=1e-7 * np.abs(ref).max())


@pytest.mark.parametrize("case", [(1, 20, 1, 1, 256, 4096, "per-step", 420), (1, 40, 1, 2, 128, 4096, "per-step", 421),
                                  (1, 70, 1, 2, 128, 1024, "chunked", 422), (1, 96, 1, 1, 128, 2048, "chunked", 423)],
                         ids=lambda c: "Dk%dDv%d-%s" % (c[4], c[5], c[6]))
def test_largest_value_head_sizes(case):
    """Value heads up to the largest size the library takes (Dv = 4096), in
    the per-step form with Dk = 256 and 128, and wide value heads in the
    chunked form (many 128-column slices per preparation block, many row
    tiles per head), against the oracle."""
    B, T, Hk, Hv, Dk, Dv, form, wid = case
    say("largest value heads", case)
    ri = rec_inputs(B, T, Hk, Hv, Dk, Dv, wid)
    y, s = gpu_recurrent_chunked(ri) if form == "chunked" else gpu_recurrent(ri)
    y_ref, s_ref = oracle_recurrent(ri)
    H.check_y(y, y_ref, str(case))
    H.check_state(s, s_ref, 1e-4, str(case))


def test_recurrent_chunked_rejects_unsupported_sizes():
    ri = rec_inputs(1, 10, 1, 1, 64, 16, 413)
    with pytest.raises(binding.GdnError):
        gpu_recurrent_chunked(ri)


def test_recurrent_chunked_long_head_drift():
    """One head of the long workload over all 32768 steps, 16 rows: the
    oracle's prologue prepares the inputs (from the head's channels only), the
    chunked recurrence runs on them, and the state stays within 1e-3."""
    say("chunked long head")
    w = inputs.WORKLOADS["long"]
    Hk, Hv, Dk, Dv = w["Hk"], w["Hv"], w["Dk"], w["Dv"]
    raw = inputs.workload("long")
    qs, ks = inputs.scales(Dk)
    b, hv, rows = 2, 21, list(range(48, 64))
    sub = H.layer_sub(raw, b, hv, rows, Hk, Hv, Dk, Dv)
    p = oracle.prep(sub["qkv"], sub["conv_w"], sub["conv_state"], sub["a"], sub["b"], sub["A_log"],
                    sub["dt_bias"], Hk=1, Hv=1, Dk=Dk, Dv=len(rows), q_scale=qs, k_scale=ks)
    ri = dict(q=oracle.round_bf16(p["q"]), k=oracle.round_bf16(p["k"]), v=oracle.round_bf16(p["v"]),
              g=oracle.round_f32(p["g"]), beta=oracle.round_f32(p["beta"]), state=sub["state"])
    y, s = gpu_recurrent_chunked(ri)
    y_ref, s_ref = oracle_recurrent(ri)
    H.check_y(y, y_ref, "long head")
    e = H.check_state(s, s_ref, 1e-3, "long head")
    say("long head state err", e)


# ------------------------------------------------------------ masked steps

def step_mask(seed, B, T, p=0.7):
    """A random step mask with runs of inactive steps (left padding on row 0)."""
    r = np.random.default_rng(seed)
    m = r.random((B, T)) < p
    m[0, : max(1, T // 5)] = False
    return m.astype(np.uint8)


MASK_CASES = [
    # B, T, Hk, Hv, Dk, Dv, wid, form
    (2, 5, 2, 4, 64, 32, 500, "per-step"),        # staging-free kernel (T < 8)
    (2, 77, 1, 2, 32, 16, 501, "per-step"),       # staged kernel, ragged chunks
    (1, 150, 2, 4, 128, 64, 502, "per-step"),
    (2, 150, 2, 4, 128, 64, 503, "chunked"),
    (3, 40, 1, 2, 128, 16, 504, "chunked"),
]


def run_form(form, ri, mask):
    return gpu_recurrent_chunked(ri, mask=mask) if form == "chunked" else gpu_recurrent(ri, mask=mask)


@pytest.mark.parametrize("case", MASK_CASES, ids=lambda c: "B%dT%dHk%dHv%dDk%dDv%d-%s" % (c[:6] + (c[7],)))
def test_masked_recurrence_matches_oracle(case):
    B, T, Hk, Hv, Dk, Dv, wid, form = case
    say("masked", case)
    ri = rec_inputs(B, T, Hk, Hv, Dk, Dv, wid)
    mask = step_mask(wid, B, T)
    y, s = run_form(form, ri, mask)
    f = oracle.bf16_to_f64
    y_ref, s_ref = oracle.recurrent(f(ri["q"]), f(ri["k"]), f(ri["v"]), ri["g"].astype(np.float64),
                                    ri["beta"].astype(np.float64), ri["state"].astype(np.float64), mask=mask)
    H.check_y(y, y_ref, str(case))
    assert not y[mask == 0].any(), "masked steps must write +0"
    e = H.check_state(s, s_ref, 1e-4, str(case))
    say("masked state err", e)


@pytest.mark.parametrize("form", ["per-step", "chunked"])
def test_mask_all_on_equals_no_mask_and_all_off_keeps_state(form):
    ri = rec_inputs(2, 70, 2, 4, 128, 32, 505)
    y, s = run_form(form, ri, None)
    y1, s1 = run_form(form, ri, np.ones((2, 70), np.uint8))
    assert np.array_equal(y, y1) and np.array_equal(s, s1)
    y0, s0 = run_form(form, ri, np.zeros((2, 70), np.uint8))
    assert not y0.any()
    assert np.array_equal(s0, ri["state"])


def test_per_step_masked_equals_run_over_active_steps():
    """Per-step form: masking steps out is bit-identical to dropping them."""
    ri = rec_inputs(2, 60, 2, 4, 64, 32, 506)
    mask = step_mask(506, 2, 60)
    y, s = gpu_recurrent(ri, mask=mask)
    for b in range(2):
        idx = np.flatnonzero(mask[b])
        assert len(idx) >= 8           # both runs take the same (staged) kernel
        sub = {k: np.ascontiguousarray(ri[k][b:b + 1, idx]) for k in ("q", "k", "v", "g", "beta")}
        yc, sc = gpu_recurrent(dict(sub, state=ri["state"][b:b + 1]))
        assert np.array_equal(yc[0], y[b, idx])
        assert np.array_equal(sc[0], s[b])


@pytest.mark.parametrize("T", [40, 96], ids=["per-step", "chunked"])
def test_masked_layer_core_matches_oracle_and_composition(T):
    B, Hk, Hv, Dk, Dv, K = 2, 2, 4, 128, 32, 4
    raw = layer_inputs(B, T, Hk, Hv, Dk, Dv, K, 507)
    qs, ks = 1.0 / Dk, Dk ** -0.5
    mask = step_mask(507, B, T)
    y, s, cs = gpu_layer_core(raw, Hk, Hv, Dk, Dv, qs, ks, mask=mask)
    p = gpu_prep(raw, Hk, Hv, Dk, Dv, qs, ks)
    cs_ref = check_core(f"masked T={T}", y, s, p, raw, Hk, Hv, Dk, Dv, qs, ks, mask=mask)
    assert np.array_equal(cs, cs_ref) and not y[mask == 0].any()
    ri = dict(q=p["q"], k=p["k"], v=p["v"], g=p["g"], beta=p["beta"], state=raw["state"])
    y2, s2 = run_form("chunked" if H.layer_uses_chunked(B, T, Hv, Dk, Dv) else "per-step", ri, mask)
    assert np.array_equal(y, y2) and np.array_equal(s, s2)
