"""binding.bind: a call marshalled once and issued again gives the same bits
as the direct call, picks up new buffer contents, and keeps its tensors
alive.  And the C ABI driven from a plain C program (tests/c_abi_demo.c)
gives the bits of the same call made through the binding."""
import numpy as np
import pytest
import torch

from linear_attention_recurrence_prep_amd import binding, inputs
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _layer(B, T, Hk, Hv, Dk, Dv, K):
    raw = inputs.layer_raw(B=B, T=T, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, K=K, workload_id=9, state=True, conv_state=True)
    d = {k: H.to_dev(raw[k]) for k in ("qkv", "conv_w", "conv_state", "a", "b", "A_log", "dt_bias", "state")}
    return raw, d


@pytest.mark.parametrize("T", [1, 96], ids=["decode", "chunked"])
def test_bound_layer_core_matches_direct(T):
    B, Hk, Hv, Dk, Dv, K = 2, 2, 4, 128, 64, 4
    raw, d = _layer(B, T, Hk, Hv, Dk, Dv, K)
    C = 2 * Hk * Dk + Hv * Dv
    qs, ks = 1.0 / Dk, Dk ** -0.5
    ws = torch.empty(max(binding.layer_core_workspace_bytes(B, T, Hk, Hv, Dk, Dv), 1), dtype=torch.uint8,
                     device=H.DEV)

    def outs():
        return (torch.empty(B, Hv, Dv, Dk, device=H.DEV), torch.empty(B, T, Hv, Dv, dtype=torch.int16, device=H.DEV),
                torch.empty(B, K - 1, C, dtype=torch.int16, device=H.DEV))

    s1, y1, c1 = outs()
    binding.layer_core(d["qkv"], d["conv_w"], d["conv_state"], c1, d["a"], d["b"], d["A_log"], d["dt_bias"],
                       d["state"], s1, y1, ws, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, q_scale=qs, k_scale=ks)
    s2, y2, c2 = outs()
    call = binding.bind(binding.layer_core, d["qkv"], d["conv_w"], d["conv_state"], c2, d["a"], d["b"],
                        d["A_log"], d["dt_bias"], d["state"], s2, y2, ws, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv,
                        q_scale=qs, k_scale=ks)
    assert isinstance(call, binding.Bound)
    torch.cuda.synchronize()
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(s1, s2) and torch.equal(c1, c2)
    # new contents of a bound input are picked up
    d["qkv"].copy_(torch.flip(d["qkv"], dims=[1]))
    call()
    binding.layer_core(d["qkv"], d["conv_w"], d["conv_state"], c1, d["a"], d["b"], d["A_log"], d["dt_bias"],
                       d["state"], s1, y1, ws, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(s1, s2) and torch.equal(c1, c2)


def test_bound_recurrent_in_place_decode_loop():
    """A bound in-place decode step issued n times equals n direct steps."""
    B, T, Hk, Hv, Dk, Dv = 3, 1, 2, 4, 64, 32
    g = torch.Generator(device="cpu").manual_seed(3)
    q = (torch.randn(B, T, Hk, Dk, generator=g) / 8).to(torch.bfloat16).to(H.DEV)
    k = (torch.randn(B, T, Hk, Dk, generator=g) / 8).to(torch.bfloat16).to(H.DEV)
    v = torch.randn(B, T, Hv, Dv, generator=g).to(torch.bfloat16).to(H.DEV)
    gg = torch.rand(B, T, Hv, generator=g).to(H.DEV)
    bb = torch.rand(B, T, Hv, generator=g).to(H.DEV)
    s0 = (torch.randn(B, Hv, Dv, Dk, generator=g) * 0.02).to(H.DEV)
    sa, sb = s0.clone(), s0.clone()
    ya = torch.empty(B, T, Hv, Dv, dtype=torch.bfloat16, device=H.DEV)
    yb = torch.empty_like(ya)
    call = binding.bind(binding.recurrent, q, k, v, gg, bb, sb, sb, yb)
    for _ in range(5):
        binding.recurrent(q, k, v, gg, bb, sa, sa, ya)
        call()
    torch.cuda.synchronize()
    assert torch.equal(sa, sb) and torch.equal(ya, yb)


@pytest.mark.parametrize("T", [20, 100], ids=["per_step", "chunked"])
def test_c_program_layer_core_matches_binding(T, tmp_path):
    """A plain C99 program (tests/c_abi_demo.c: hipMalloc, hipMemcpy and one
    gdn_layer_core call on the null stream, no Python in between) gives the
    bits of the same call made through the Python binding."""
    import os
    import subprocess
    from linear_attention_recurrence_prep_amd import build as bld
    demo = bld.C_DEMO
    assert os.path.exists(demo), "the C test program is built by build()"
    B, Hk, Hv, Dk, Dv, K = 2, 2, 4, 128, 64, 4
    raw, d = _layer(B, T, Hk, Hv, Dk, Dv, K)
    for name in ("qkv", "conv_w", "conv_state", "a", "b", "A_log", "dt_bias", "state"):
        np.ascontiguousarray(raw[name]).tofile(tmp_path / name)
    qs, ks = 1.0 / Dk, Dk ** -0.5
    print("[case] C program layer core", T, flush=True)
    r = subprocess.run([demo, "run", str(tmp_path), str(B), str(T), str(Hk), str(Hv), str(Dk), str(Dv), str(K),
                        repr(qs), repr(ks)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    C = 2 * Hk * Dk + Hv * Dv
    y_c = np.fromfile(tmp_path / "y", dtype=np.int16).reshape(B, T, Hv, Dv)
    s_c = np.fromfile(tmp_path / "state_out", dtype=np.float32).reshape(B, Hv, Dv, Dk)
    cs_c = np.fromfile(tmp_path / "conv_state_out", dtype=np.int16).reshape(B, K - 1, C)
    ws = torch.empty(max(binding.layer_core_workspace_bytes(B, T, Hk, Hv, Dk, Dv), 1), dtype=torch.uint8,
                     device=H.DEV)
    s = torch.empty(B, Hv, Dv, Dk, device=H.DEV)
    y = torch.empty(B, T, Hv, Dv, dtype=torch.int16, device=H.DEV)
    cs = torch.empty(B, K - 1, C, dtype=torch.int16, device=H.DEV)
    binding.layer_core(d["qkv"], d["conv_w"], d["conv_state"], cs, d["a"], d["b"], d["A_log"], d["dt_bias"],
                       d["state"], s, y, ws, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), y_c)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_c.view(np.uint32))
    assert np.array_equal(cs.cpu().numpy(), cs_c)
