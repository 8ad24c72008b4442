"""Tensors past 2^31 elements: every offset into qkv, v, y, the chunk
workspace and the state is 64-bit.  A batched call whose later sequences sit
beyond element 2^31 of their tensors must give, for each such sequence, the
bits of a one-sequence call on that sequence's own slices (where every offset
stays small): the arithmetic per sequence does not depend on the batch, so
any truncated offset shows as a mismatch.  Inputs are seeded and drawn on the
device with the workloads' distributions (qkv, a, b N(0, 1); conv weights
N(0, 0.1^2); A_log = log U[1, 16]; dt_bias N(0, 0.1^2); state N(0, 0.02^2);
a random conv state).  About 60 GB of device memory at most; skipped on a
device with less free."""
import sys

import pytest
import torch

from linear_attention_recurrence_prep_amd import binding, inputs
from tests import helpers as H

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
NAN_BF16 = 0x7FC0
HK, HV, DK, DV, K = 16, 32, 128, 128, 4
C = 2 * HK * DK + HV * DV
# one sequence of qkv stays below 2^31 elements, three go past it (and the
# y and v tensors of three sequences too)
T_LONG = 196608
B_LONG = 3
# the decode batch whose state passes 2^31 elements (2^19 per sequence)
B_DEC = 4100


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def need_free(nbytes):
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info(DEV)
    if free < nbytes:
        pytest.skip(f"needs {nbytes / 2**30:.0f} GiB of free device memory, {free / 2**30:.0f} GiB free")


@pytest.fixture(autouse=True)
def _release():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def device_inputs(B, T, seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    bf = dict(dtype=torch.bfloat16, device=DEV, generator=gen)
    f32 = dict(dtype=torch.float32, device=DEV, generator=gen)
    d = {
        "qkv": torch.randn(B, T, C, **bf),
        "conv_w": torch.randn(C, K, **f32).mul_(0.1).to(torch.bfloat16),
        "conv_state": torch.randn(B, K - 1, C, **bf),
        "a": torch.randn(B, T, HV, **bf),
        "b": torch.randn(B, T, HV, **bf),
        "A_log": torch.rand(HV, **f32).mul_(15).add_(1).log_(),
        "dt_bias": torch.randn(HV, **f32).mul_(0.1),
        "state": torch.randn(B, HV, DV, DK, **f32).mul_(0.02),
    }
    return d


def run_layer_core(d, sl, ws):
    """gdn_layer_core on the sequences sl of d; returns (y, state, conv state)."""
    x = {k: (v[sl] if k in ("qkv", "conv_state", "a", "b", "state") else v) for k, v in d.items()}
    B, T = x["qkv"].shape[:2]
    y = torch.full((B, T, HV, DV), NAN_BF16, dtype=torch.int16, device=DEV)
    s = torch.full((B, HV, DV, DK), float("nan"), dtype=torch.float32, device=DEV)
    cs = torch.empty(B, K - 1, C, dtype=torch.int16, device=DEV)
    qs, ks = inputs.scales(DK)
    assert ws.numel() >= binding.layer_core_workspace_bytes(B, T, HK, HV, DK, DV)
    binding.layer_core(x["qkv"], x["conv_w"], x["conv_state"], cs, x["a"], x["b"], x["A_log"], x["dt_bias"],
                       x["state"], s, y, ws, Hk=HK, Hv=HV, Dk=DK, Dv=DV, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    return y, s, cs


def test_layer_core_prefill_past_2_31_elements():
    """Chunked layer core, B = 3, T = 196608: qkv (4.8e9 elements), v and y
    (2.4e9) pass 2^31 inside sequence 1; the workspace is 27 GB.  Sequences
    1 and 2 equal one-sequence calls bit for bit, and the whole batch equals
    gdn_prep followed by gdn_recurrent_chunked bit for bit."""
    B, T = B_LONG, T_LONG
    assert B * T * C > 2**31 > T * C and B * T * HV * DV > 2**31
    assert H.layer_uses_chunked(B, T, HV, DK, DV) and H.layer_uses_chunked(1, T, HV, DK, DV)
    nws = binding.layer_core_workspace_bytes(B, T, HK, HV, DK, DV)
    assert nws == binding.recurrent_chunked_workspace_bytes(B, T, HK, HV, DK, DV)
    # qkv + y (layer core and composition) + q, k, v + workspace, with room
    need = 2 * B * T * C + 2 * (2 * B * T * HV * DV) + 2 * B * T * (2 * HK * DK + HV * DV) + nws
    need_free(int(need * 1.25))
    say("layer core past 2^31 elements", B, T)
    d = device_inputs(B, T, 2031)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    y, s, cs = run_layer_core(d, slice(0, B), ws)
    assert not (y == NAN_BF16).any().item(), "y not written everywhere"
    assert torch.isfinite(s).all().item()

    say("one-sequence calls")
    for b in (1, 2):
        y1, s1, cs1 = run_layer_core(d, slice(b, b + 1), ws)
        assert torch.equal(y1[0], y[b]), f"sequence {b}: y differs from its one-sequence call"
        assert torch.equal(s1[0], s[b]), f"sequence {b}: state differs from its one-sequence call"
        assert torch.equal(cs1[0], cs[b]), f"sequence {b}: conv state differs from its one-sequence call"
        del y1, s1, cs1

    say("composition gdn_prep + gdn_recurrent_chunked")
    q = torch.empty(B, T, HK, DK, dtype=torch.int16, device=DEV)
    k = torch.empty_like(q)
    v = torch.empty(B, T, HV, DV, dtype=torch.int16, device=DEV)
    g = torch.empty(B, T, HV, dtype=torch.float32, device=DEV)
    beta = torch.empty_like(g)
    cs2 = torch.empty_like(cs)
    qs, ks = inputs.scales(DK)
    binding.prep(d["qkv"], d["conv_w"], d["conv_state"], cs2, d["a"], d["b"], d["A_log"], d["dt_bias"],
                 q, k, v, g, beta, Hk=HK, Hv=HV, Dk=DK, Dv=DV, q_scale=qs, k_scale=ks)
    state = d["state"]
    del d
    y2 = torch.full_like(y, NAN_BF16)
    s2 = torch.full_like(s, float("nan"))
    binding.recurrent_chunked(q, k, v, g, beta, state, s2, y2, ws)
    torch.cuda.synchronize()
    assert torch.equal(cs2, cs), "conv state differs from gdn_prep's"
    assert torch.equal(s2, s), "state differs from the composition"
    assert torch.equal(y2, y), "y differs from the composition"


@pytest.mark.parametrize("T", [1, 12, 64], ids=["decode", "per_step_T12", "chunked_T64"])
def test_state_past_2_31_elements(T):
    """The layer core at B = 4100: the state holds 2.15e9 elements, so
    sequences from 4096 on sit past 2^31.  T = 1 takes the single-step
    kernel, T = 12 the per-step form with staged chunks, T = 64 the chunked
    form (fused preparation, two waves per state tile).  Sequences 4095 and
    4099 equal one-sequence calls bit for bit."""
    B = B_DEC
    n_state = B * HV * DV * DK
    assert n_state > 2**31 > 4096 * HV * DV * DK - 1
    assert H.layer_uses_chunked(B, T, HV, DK, DV) == (T >= 64) == H.layer_uses_chunked(1, T, HV, DK, DV)
    nws = binding.layer_core_workspace_bytes(B, T, HK, HV, DK, DV)
    need = 8 * n_state + 2 * B * T * C + 2 * B * T * HV * DV + nws
    need_free(int(need * 1.25))
    say("state past 2^31 elements", B, T)
    d = device_inputs(B, T, 2032 + T)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=DEV)
    y, s, cs = run_layer_core(d, slice(0, B), ws)
    assert not (y == NAN_BF16).any().item(), "y not written everywhere"
    for b in (4095, 4099):
        say("one-sequence call", b)
        y1, s1, cs1 = run_layer_core(d, slice(b, b + 1), ws)
        assert torch.equal(y1[0], y[b]), f"sequence {b}: y differs from its one-sequence call"
        assert torch.equal(s1[0], s[b]), f"sequence {b}: state differs from its one-sequence call"
        assert torch.equal(cs1[0], cs[b]), f"sequence {b}: conv state differs from its one-sequence call"


def test_gated_rmsnorm_past_2_31_elements():
    """Output epilogue over y and z of 2.4e9 elements each (B = 3,
    T = 196608): sequence 2 equals a one-sequence call bit for bit."""
    B, T = B_LONG, T_LONG
    n = B * T * HV * DV
    assert n > 2**31
    need_free(int(3 * 2 * n * 1.1))
    say("gated rmsnorm past 2^31 elements", B, T)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(2033)
    y = torch.randn(B, T, HV, DV, dtype=torch.bfloat16, device=DEV, generator=gen)
    z = torch.randn(B, T, HV, DV, dtype=torch.bfloat16, device=DEV, generator=gen)
    w = torch.randn(DV, dtype=torch.float32, device=DEV, generator=gen).add_(1).to(torch.bfloat16)
    out = torch.full((B, T, HV, DV), NAN_BF16, dtype=torch.int16, device=DEV)
    binding.gated_rmsnorm(y, z, w, out)
    torch.cuda.synchronize()
    assert not (out == NAN_BF16).any().item(), "out not written everywhere"
    out1 = torch.full((1, T, HV, DV), NAN_BF16, dtype=torch.int16, device=DEV)
    binding.gated_rmsnorm(y[2:3], z[2:3], w, out1)
    torch.cuda.synchronize()
    assert torch.equal(out1[0], out[2]), "sequence 2 differs from its one-sequence call"


def unit_rows(x):
    """Rows scaled to unit norm over the last axis (keys as the prologue's
    normalisation leaves them), stored as bf16."""
    xf = x.float()
    return (xf / xf.norm(dim=-1, keepdim=True).clamp_min(1e-6)).to(torch.bfloat16)


def recurrence_inputs(B, T, seed, per_key):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    bf = dict(dtype=torch.bfloat16, device=DEV, generator=gen)
    f32 = dict(dtype=torch.float32, device=DEV, generator=gen)
    gshape = (B, T, HV, DK) if per_key else (B, T, HV)
    return {
        "q": unit_rows(torch.randn(B, T, HK, DK, **bf)),
        "k": unit_rows(torch.randn(B, T, HK, DK, **bf)),
        "v": torch.randn(B, T, HV, DV, **bf),
        "g": torch.rand(*gshape, **f32).mul_(0.7).add_(0.3),
        "beta": torch.rand(B, T, HV, **f32),
        "state": torch.randn(B, HV, DV, DK, **f32).mul_(0.02),
    }


def test_per_key_chunked_past_2_31_elements():
    """The chunked recurrence with the per-key gate at B = 3, T = 196608: the
    gate rows (2.4e9 elements), v and y pass 2^31 inside sequence 1, the
    workspace is about 40 GB.  Sequences 1 and 2 equal one-sequence calls bit
    for bit."""
    B, T = B_LONG, T_LONG
    ng = B * T * HV * DK
    assert ng > 2**31 and B * T * HV * DV > 2**31
    nws = binding.recurrent_chunked_per_key_workspace_bytes(B, T, HK, HV, DK, DV)
    need = 4 * ng + 2 * (2 * B * T * HK * DK) + 2 * (2 * B * T * HV * DV) + 2 * T * HV * DV + nws
    need_free(int(need * 1.25))
    say("per-key chunked past 2^31 elements", B, T)
    d = recurrence_inputs(B, T, 2041, per_key=True)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)

    def run(sl):
        x = {k_: v_[sl] for k_, v_ in d.items()}
        n = x["q"].shape[0]
        y = torch.full((n, T, HV, DV), NAN_BF16, dtype=torch.int16, device=DEV)
        s = torch.full((n, HV, DV, DK), float("nan"), dtype=torch.float32, device=DEV)
        binding.recurrent_chunked_per_key(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state"], s, y, ws)
        torch.cuda.synchronize()
        return y, s

    y, s = run(slice(0, B))
    assert not (y == NAN_BF16).any().item(), "y not written everywhere"
    assert torch.isfinite(s).all().item()
    for b in (1, 2):
        say("one-sequence call", b)
        y1, s1 = run(slice(b, b + 1))
        assert torch.equal(y1[0], y[b]), f"sequence {b}: y differs from its one-sequence call"
        assert torch.equal(s1[0], s[b]), f"sequence {b}: state differs from its one-sequence call"
        del y1, s1


@pytest.mark.parametrize("per_key", [False, True], ids=["per_head_gate", "per_key_gate"])
def test_snapshots_past_2_31_elements(per_key):
    """gdn_recurrent_snapshots at B = 4100, T = 2 with the state after steps 1
    and 2: the state and each snapshot hold 2.15e9 elements.  Sequences 4095
    and 4099 equal one-sequence calls bit for bit, snapshots included."""
    B, T = B_DEC, 2
    n_state = B * HV * DV * DK
    assert n_state > 2**31
    steps = [1, 2]
    need_free(int(4 * n_state * (2 + len(steps)) * 1.25))
    say("snapshots past 2^31 elements", B, "per-key" if per_key else "per-head")
    d = recurrence_inputs(B, T, 2042 + per_key, per_key)

    def run(sl):
        x = {k_: v_[sl] for k_, v_ in d.items()}
        n = x["q"].shape[0]
        y = torch.full((n, T, HV, DV), NAN_BF16, dtype=torch.int16, device=DEV)
        s = torch.full((n, HV, DV, DK), float("nan"), dtype=torch.float32, device=DEV)
        snaps = torch.full((len(steps), n, HV, DV, DK), float("nan"), dtype=torch.float32, device=DEV)
        binding.recurrent_snapshots(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state"], s, y, steps, snaps)
        torch.cuda.synchronize()
        return y, s, snaps

    y, s, snaps = run(slice(0, B))
    assert not (y == NAN_BF16).any().item(), "y not written everywhere"
    assert torch.equal(snaps[-1], s), "the snapshot after the last step is the final state"
    for b in (4095, 4099):
        say("one-sequence call", b)
        y1, s1, sn1 = run(slice(b, b + 1))
        assert torch.equal(y1[0], y[b]), f"sequence {b}: y differs from its one-sequence call"
        assert torch.equal(s1[0], s[b]), f"sequence {b}: state differs from its one-sequence call"
        assert torch.equal(sn1[:, 0], snaps[:, b]), f"sequence {b}: snapshots differ from its one-sequence call"
