"""GPU parity of the output epilogue (gated RMS normalisation of the
recurrence output) and of the gated layer core, through the C ABI, against
the CPU oracle on the same seeded inputs.  Bar: within one bf16 ulp of the
fp64 value with at least 99% correctly rounded (tests/helpers.py,
check_epilogue); in-place and composed calls bit for bit."""
import sys

import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrence_prep_amd import binding, inputs
from tests import helpers as H
from tests.test_parity_gpu import gpu_layer_core, gpu_prep, layer_inputs, oracle_on_gpu_prologue

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.lib()
    yield
    torch.cuda.synchronize()


def gpu_gated(y, z, w, eps, out="new"):
    dy, dz, dw = H.to_dev(y), H.to_dev(z), H.to_dev(w)
    if out == "y":
        o = dy
    elif out == "z":
        o = dz
    else:
        full, o = H.guarded(y.shape, torch.int16, NAN_BF16)
    binding.gated_rmsnorm(dy, dz, dw, o, eps=eps)
    torch.cuda.synchronize()
    if out == "new":
        assert H.guards_intact(full, NAN_BF16), "guard band written"
    return H.bits(o)


EPI_CASES = [
    # B, T, Hv, Dv, wid      lanes per row / vectors per lane
    (1, 64, 4, 128, 600),    # 16 / 1 (the layer's shape)
    (2, 37, 3, 24, 601),     # 4 / 1, one idle lane per row
    (1, 5, 2, 8, 602),       # 1 / 1
    (2, 33, 2, 48, 603),     # 8 / 1, two idle lanes
    (1, 9, 1, 520, 604),     # 64 / 2, ragged second vector
    (1, 3, 2, 4096, 605),    # 64 / 8 (largest Dv)
    (1, 1, 1, 16, 606),      # 2 / 1, one row
    (1, 17, 5, 256, 607),    # 32 / 1, partial last block
]


@pytest.mark.parametrize("case", EPI_CASES, ids=lambda c: "B%dT%dHv%dDv%d" % c[:4])
@pytest.mark.parametrize("eps", [1e-6, 0.25])
def test_gated_rmsnorm_matches_oracle(case, eps):
    B, T, Hv, Dv, wid = case
    say("gated_rmsnorm", case, eps)
    r = inputs.epilogue_raw(B=B, T=T, Hv=Hv, Dv=Dv, workload_id=wid)
    out = gpu_gated(r["y"], r["z"], r["norm_weight"], eps)
    ref = oracle.gated_rmsnorm(r["y"], r["z"], r["norm_weight"], eps=eps)
    flips = H.check_epilogue(out, ref, str(case))
    say("flips", flips, "of", out.size)


def test_gated_rmsnorm_extremes():
    """Gate arguments across silu's range (exp overflow and underflow, signed
    zeros), all-zero rows, eps-dominated rows, negative weights, eps = 0."""
    B, T, Hv, Dv = 2, 12, 3, 64
    r = inputs.epilogue_raw(B=B, T=T, Hv=Hv, Dv=Dv, workload_id=610)
    f = oracle.bf16_to_f64
    zf = f(r["z"])
    special = np.array([0.0, -0.0, 1e-30, -1e-30, 20.0, -20.0, 87.0, -87.0, 89.0, -89.0, 100.0, -100.0,
                        -200.0, 6e4, -3e38, 1.0])
    zf[0, :, :, :16] = special
    yf = f(r["y"])
    yf[1, 3, 1] = 0.0                       # all-zero row
    yf[1, 4, 2] *= 2.0 ** -30               # eps dominates
    yf[0, 5, 0, ::2] = -yf[0, 5, 0, ::2]
    wf = f(r["norm_weight"])
    wf[::5] = -wf[::5]
    y, z, w = oracle.round_bf16(yf), oracle.round_bf16(zf), oracle.round_bf16(wf)
    for eps in (1e-6, 0.0):
        if eps == 0.0:
            y = y.copy()
            y[1, 3, 1] = oracle.round_bf16(np.full(Dv, 0.5))   # eps = 0 with a zero row is NaN by definition
        out = gpu_gated(y, z, w, eps)
        ref = oracle.gated_rmsnorm(y, z, w, eps=eps)
        H.check_epilogue(out, ref, f"eps={eps}")
        if eps:
            assert not oracle.bf16_to_f64(out[1, 3, 1]).any()


def test_gated_rmsnorm_in_place_and_repeat():
    r = inputs.epilogue_raw(B=2, T=21, Hv=4, Dv=128, workload_id=611)
    a = gpu_gated(r["y"], r["z"], r["norm_weight"], 1e-6)
    assert np.array_equal(gpu_gated(r["y"], r["z"], r["norm_weight"], 1e-6, out="y"), a)
    assert np.array_equal(gpu_gated(r["y"], r["z"], r["norm_weight"], 1e-6, out="z"), a)
    assert np.array_equal(gpu_gated(r["y"], r["z"], r["norm_weight"], 1e-6), a)


def test_gated_rmsnorm_prefill_workload_full_size():
    """The epilogue at the prefill workload's size (B=1, T=4096, Hv=32,
    Dv=128), every value against the oracle, in the launch configuration the
    benchmark times."""
    w = inputs.WORKLOADS["prefill"]
    r = inputs.epilogue_raw(B=1, T=w["T"], Hv=w["Hv"], Dv=w["Dv"], workload_id=w["id"])
    out = gpu_gated(r["y"], r["z"], r["norm_weight"], 1e-6)
    ref = oracle.gated_rmsnorm(r["y"], r["z"], r["norm_weight"], eps=1e-6)
    flips = H.check_epilogue(out, ref, "prefill")
    say("prefill epilogue flips", flips, "of", out.size)


def gpu_layer_core_gated(raw, gate, Hk, Hv, Dk, Dv, qs, ks, eps=1e-6, norm_eps=1e-6, mask=None):
    B, T, C = raw["qkv"].shape
    K = raw["conv_w"].shape[1]
    d = {k: H.to_dev(raw[k]) for k in ("qkv", "conv_w", "conv_state", "a", "b", "A_log", "dt_bias", "state")}
    z, w = H.to_dev(gate["z"]), H.to_dev(gate["norm_weight"])
    s_out = torch.empty(B, Hv, Dv, Dk, dtype=torch.float32, device=H.DEV)
    full, out = H.guarded((B, T, Hv, Dv), torch.int16, NAN_BF16)
    cs_out = torch.empty(B, K - 1, C, dtype=torch.int16, device=H.DEV)
    nws = binding.layer_core_workspace_bytes(B, T, Hk, Hv, Dk, Dv)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=H.DEV)
    m = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).to(H.DEV)
    binding.layer_core_gated(d["qkv"], d["conv_w"], d["conv_state"], cs_out, d["a"], d["b"], d["A_log"],
                             d["dt_bias"], z, w, d["state"], s_out, out, ws, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv,
                             q_scale=qs, k_scale=ks, eps=eps, norm_eps=norm_eps, mask=m)
    torch.cuda.synchronize()
    assert H.guards_intact(full, NAN_BF16)
    return H.bits(out), H.f32(s_out), H.bits(cs_out)


def check_end_to_end(out_bits, y_ref, gate, eps):
    """out against the oracle's composition (its y rounded to bf16, then the
    epilogue), with the bound that y's own tolerance implies: if each y value
    may be off by e_i <= 1.5 ulp(y) + 1e-3 (1 ulp + 1e-3 for the GPU's y, half
    an ulp for the oracle's rounding), then with c = silu(z) w and r the row's
    rms, |d out_i| <= (|c_i| e_i + |out_i| rms(e)) / (r - rms(e)), plus one
    ulp of out for its rounding."""
    yb = oracle.round_bf16(y_ref)
    ref = oracle.gated_rmsnorm(yb, gate["z"], gate["norm_weight"], eps=eps)
    f = oracle.bf16_to_f64
    yr = f(yb)
    e = 1.5 * H.bf16_ulp(y_ref) + 1e-3
    zf, wf = f(gate["z"]), f(gate["norm_weight"])
    c = np.abs(zf / (1.0 + np.exp(-zf)) * wf)
    r = np.sqrt(np.mean(yr * yr, -1, keepdims=True) + eps)
    re = np.sqrt(np.mean(e * e, -1, keepdims=True))
    denom = np.maximum(r - re, 1e-300)
    bound = (c * e + np.abs(ref) * re) / denom + H.bf16_ulp(ref)
    err = np.abs(f(out_bits) - ref)
    assert not np.isnan(f(out_bits)).any()
    assert (err <= bound).all(), f"{(err > bound).sum()} values beyond the implied bound"
    return float(np.max(err / bound))


@pytest.mark.parametrize("T", [40, 96], ids=["per-step", "chunked"])
def test_layer_core_gated_matches_oracle_and_composition(T):
    B, Hk, Hv, Dk, Dv, K = 2, 2, 4, 128, 64, 4
    raw = layer_inputs(B, T, Hk, Hv, Dk, Dv, K, 620, state=True)
    gate = inputs.epilogue_raw(B=B, T=T, Hv=Hv, Dv=Dv, workload_id=620, with_y=False)
    qs, ks = 1.0 / Dk, Dk ** -0.5
    mask = (np.arange(T)[None, :] >= np.array([[0], [T // 3]])).astype(np.uint8)   # left padding
    out, s, cs = gpu_layer_core_gated(raw, gate, Hk, Hv, Dk, Dv, qs, ks, mask=mask)
    # composition: the layer core, then the epilogue, bit for bit
    y2, s2, cs2 = gpu_layer_core(raw, Hk, Hv, Dk, Dv, qs, ks, mask=mask)
    out2 = gpu_gated(y2, gate["z"], gate["norm_weight"], 1e-6)
    assert np.array_equal(out, out2) and np.array_equal(s, s2) and np.array_equal(cs, cs2)
    # the oracle's composition: its recurrence on the device's prologue
    # outputs (state 1e-4), its layer core then the epilogue (output within
    # the bound y's tolerance implies)
    p = gpu_prep(raw, Hk, Hv, Dk, Dv, qs, ks)
    _, s_r = oracle_on_gpu_prologue(p, raw["state"], mask)
    e = H.check_state(s, s_r, 1e-4, f"T={T}")
    y_ref, _, _ = oracle.layer_core(raw["qkv"], raw["conv_w"], raw["conv_state"], raw["a"], raw["b"],
                                    raw["A_log"], raw["dt_bias"], raw["state"], Hk=Hk, Hv=Hv, Dk=Dk,
                                    Dv=Dv, q_scale=qs, k_scale=ks, mask=mask)
    worst = check_end_to_end(out, y_ref, gate, 1e-6)
    say("gated layer core: worst error / bound", worst, "state err", e)


def test_layer_core_gated_prefill_workload_sampled_heads():
    """The gated layer core at the prefill workload's full size; two whole
    v-heads recomputed end to end by the oracle."""
    w = inputs.WORKLOADS["prefill"]
    Hk, Hv, Dk, Dv, T = w["Hk"], w["Hv"], w["Dk"], w["Dv"], w["T"]
    raw = inputs.workload("prefill")
    gate = inputs.epilogue_raw(B=1, T=T, Hv=Hv, Dv=Dv, workload_id=w["id"], with_y=False)
    qs, ks = inputs.scales(Dk)
    out, s, _ = gpu_layer_core_gated(raw, gate, Hk, Hv, Dk, Dv, qs, ks)
    for hv in (3, 26):
        sub = H.layer_sub(raw, 0, hv, list(range(Dv)), Hk, Hv, Dk, Dv)
        y_ref, _, _ = oracle.layer_core(sub["qkv"], sub["conv_w"], sub["conv_state"], sub["a"], sub["b"],
                                        sub["A_log"], sub["dt_bias"], sub["state"], Hk=1, Hv=1, Dk=Dk,
                                        Dv=Dv, q_scale=qs, k_scale=ks)
        g = dict(z=np.ascontiguousarray(gate["z"][:, :, hv:hv + 1]), norm_weight=gate["norm_weight"])
        worst = check_end_to_end(np.ascontiguousarray(out[:, :, hv:hv + 1]), y_ref, g, 1e-6)
        say("prefill gated hv", hv, "worst error / bound", worst)
