"""The allocation-free layer core (gdn_layer_core_no_alloc, the library's own
device scratch as workspace) against gdn_layer_core_masked with a caller
workspace: the same kernels, so the same bits, over consecutive calls that
share the scratch (each later call smaller than the first, on a different
path through the layer core)."""
import sys

import numpy as np
import pytest
import torch

from linear_attention_recurrence_prep_amd import binding, inputs
from tests import helpers as H

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.lib()
    yield
    torch.cuda.synchronize()


def run(raw, shape, mask, no_alloc, cs_in_place):
    B, T, Hk, Hv, Dk, Dv, K = shape
    C = 2 * Hk * Dk + Hv * Dv
    d = {k: H.to_dev(raw[k]) for k in ("qkv", "conv_w", "conv_state", "a", "b", "A_log", "dt_bias", "state")}
    y = torch.full((B, T, Hv, Dv), 0x7FC0, dtype=torch.int16, device=H.DEV)
    s_out = torch.full((B, Hv, Dv, Dk), float("nan"), dtype=torch.float32, device=H.DEV)
    cs_out = d["conv_state"] if cs_in_place else torch.empty(B, K - 1, C, dtype=torch.int16, device=H.DEV)
    m = None if mask is None else torch.from_numpy(mask).to(H.DEV)
    kw = dict(Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, q_scale=1.0 / Dk, k_scale=Dk ** -0.5, mask=m)
    common = (d["qkv"], d["conv_w"], d["conv_state"], cs_out, d["a"], d["b"], d["A_log"], d["dt_bias"],
              d["state"], s_out, y)
    if no_alloc:
        binding.layer_core_no_alloc(*common, **kw)
    else:
        nws = binding.layer_core_workspace_bytes(B, T, Hk, Hv, Dk, Dv)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=H.DEV)
        binding.layer_core(*common, ws, **kw)
    torch.cuda.synchronize()
    return H.bits(y), H.f32(s_out), H.bits(cs_out)


# B, T, Hk, Hv, Dk, Dv, K, masked, conv state in place
CALLS = [
    (2, 300, 4, 8, 128, 128, 4, True, False),    # chunked form, prologue fused into its preparation
    (1, 100, 2, 8, 128, 64, 3, False, True),     # smaller: fused, GQA 4 with the conv state in place
    (1, 40, 2, 4, 64, 32, 4, True, False),       # smaller again: prologue, then the per-step form
]


def test_no_alloc_matches_caller_workspace_over_consecutive_calls():
    nws = [binding.layer_core_workspace_bytes(*c[:6]) for c in CALLS]
    assert nws[0] > nws[1] > nws[2] > 0 and nws[0] <= binding.NO_ALLOC_SCRATCH_BYTES
    for i, c in enumerate(CALLS):
        shape, masked, ip = c[:7], c[7], c[8]
        say("no_alloc call", i, shape, "masked" if masked else "", "conv state in place" if ip else "")
        raw = inputs.layer_raw(B=shape[0], T=shape[1], Hk=shape[2], Hv=shape[3], Dk=shape[4], Dv=shape[5],
                               K=shape[6], workload_id=900 + i, state=True, conv_state=True)
        mask = None
        if masked:
            r = np.random.default_rng(900 + i)
            mask = (r.random(shape[:2]) < 0.8).astype(np.uint8)
        y1, s1, cs1 = run(raw, shape, mask, True, ip)
        y0, s0, cs0 = run(raw, shape, mask, False, ip)
        assert np.array_equal(y1, y0), f"call {i}: y differs"
        assert np.array_equal(s1, s0), f"call {i}: state differs"
        assert np.array_equal(cs1, cs0), f"call {i}: conv state differs"
        assert not np.isnan(s1).any()


def test_no_alloc_empty_batch_and_size_limit():
    say("no_alloc B=0 / size limit")
    Hk, Hv, Dk, Dv, K = 16, 32, 128, 128, 4
    C = 2 * Hk * Dk + Hv * Dv
    dev = H.DEV
    # B = 0: sets the device up, launches nothing
    e = lambda *s, dt=torch.int16: torch.empty(*s, dtype=dt, device=dev)
    binding.layer_core_no_alloc(e(0, 8, C), e(C, K), None, None, e(0, 8, Hv), e(0, 8, Hv),
                                e(Hv, dt=torch.float32), e(Hv, dt=torch.float32), None,
                                e(0, Hv, Dv, Dk, dt=torch.float32), e(0, 8, Hv, Dv), Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv,
                                q_scale=1.0, k_scale=1.0)
    # a prefill longer than the scratch holds is refused before any launch
    T = 4096
    assert binding.layer_core_workspace_bytes(1, T, Hk, Hv, Dk, Dv) > binding.NO_ALLOC_SCRATCH_BYTES
    with pytest.raises(binding.GdnError) as ei:
        binding.layer_core_no_alloc(e(1, T, C), e(C, K), None, None, e(1, T, Hv), e(1, T, Hv),
                                    e(Hv, dt=torch.float32), e(Hv, dt=torch.float32), None,
                                    e(1, Hv, Dv, Dk, dt=torch.float32), e(1, T, Hv, Dv), Hk=Hk, Hv=Hv, Dk=Dk,
                                    Dv=Dv, q_scale=1.0, k_scale=1.0)
    assert ei.value.status == -6
    torch.cuda.synchronize()
