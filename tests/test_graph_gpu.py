"""Capture of the library's calls in a HIP graph (torch.cuda.CUDAGraph):
a decode loop of layer-core steps (state and conv state updated in place,
then the output epilogue) is captured once and replayed several times, with
eager work and synchronisation between the replays; every replay must give
the eager run's outputs bit for bit.  The calls enqueue kernels only (no
memset, no allocation, no synchronisation), which is what makes them
capturable."""
import numpy as np
import pytest
import torch

from linear_attention_recurrence_prep_amd import binding, inputs
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.lib()
    yield
    torch.cuda.synchronize()


def test_decode_loop_graph_replays_match_eager():
    B, T, Hk, Hv, Dk, Dv, K, STEPS = 4, 1, 2, 4, 128, 64, 4, 6
    qs, ks = inputs.scales(Dk)
    raws = [inputs.layer_raw(B=B, T=T, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, K=K, workload_id=800 + i, state=True,
                             conv_state=True) for i in range(STEPS)]
    gate = inputs.epilogue_raw(B=B, T=T, Hv=Hv, Dv=Dv, workload_id=800, with_y=False)
    common = {k: H.to_dev(raws[0][k]) for k in ("conv_w", "A_log", "dt_bias")}
    per = [{k: H.to_dev(r[k]) for k in ("qkv", "a", "b")} for r in raws]
    z = [H.to_dev(inputs.epilogue_raw(B=B, T=T, Hv=Hv, Dv=Dv, workload_id=810 + i, with_y=False)["z"])
         for i in range(STEPS)]
    w = H.to_dev(gate["norm_weight"])
    st0 = H.to_dev(raws[0]["state"])
    cs0 = H.to_dev(raws[0]["conv_state"])
    st, cs = st0.clone(), cs0.clone()
    outs = [torch.empty(B, T, Hv, Dv, dtype=torch.int16, device=H.DEV) for _ in range(STEPS)]
    ws = torch.empty(max(binding.layer_core_workspace_bytes(B, T, Hk, Hv, Dk, Dv), 1), dtype=torch.uint8,
                     device=H.DEV)

    def loop():
        for i in range(STEPS):
            p = per[i]
            binding.layer_core_gated(p["qkv"], common["conv_w"], cs, cs, p["a"], p["b"], common["A_log"],
                                     common["dt_bias"], z[i], w, st, st, outs[i], ws, Hk=Hk, Hv=Hv, Dk=Dk,
                                     Dv=Dv, q_scale=qs, k_scale=ks)

    # eager reference
    loop()
    torch.cuda.synchronize()
    ref = ([H.bits(o) for o in outs], H.f32(st), H.bits(cs))

    # capture on a side stream (default priority), after a warm-up there
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.copy_(st0)
        cs.copy_(cs0)
        loop()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        loop()
    torch.cuda.synchronize()

    for rep in range(4):
        st.copy_(st0)
        cs.copy_(cs0)
        for o in outs:
            o.fill_(0x7FC0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = ([H.bits(o) for o in outs], H.f32(st), H.bits(cs))
        for a_, b_ in zip(got[0], ref[0]):
            assert np.array_equal(a_, b_), f"replay {rep}: output differs"
        assert np.array_equal(got[1], ref[1]) and np.array_equal(got[2], ref[2]), f"replay {rep}: state differs"
        # eager work between replays
        tmp = torch.empty_like(outs[0])
        binding.gated_rmsnorm(outs[0], z[0], w, tmp)
        torch.cuda.synchronize()
