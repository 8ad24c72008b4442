"""GPU parity over a seeded sweep of random valid shapes (batch, length, head
counts and sizes, GQA group, conv width, with and without conv / recurrent
state and step masks): the layer core against the oracle's recurrence on the
device's own prologue outputs (strict y bounds, state 1e-4 per head) and
against the oracle's own prologue, conv state bit-exact, and bit for bit
against the prologue followed by the recurrence entry point it is defined as
(chunked or per-step by the rule of tests.helpers.layer_uses_chunked)."""
import numpy as np
import pytest

from tests import helpers as H
from tests.test_parity_gpu import (check_core, gpu_layer_core, gpu_prep, gpu_recurrent, gpu_recurrent_chunked,
                                   layer_inputs, say, step_mask)

pytestmark = pytest.mark.gpu


def sweep_shapes(n, seed, chunked_only=False, max_work=4e7):
    """n random valid shapes (B, T, Hk, Hv, Dk, Dv, K, state, conv_state, masked)
    whose recurrence work B*T*Hv*Dk*Dv stays small enough for the oracle;
    chunked_only draws only shapes the layer core runs in the chunked form."""
    r = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        Dk = 128 if chunked_only else int(r.choice([32, 64, 128, 256]))
        Hk = int(r.integers(1, 4))
        Hv = Hk * int(r.integers(1, 5))
        Dv = 8 * int(r.integers(1, 33)) if r.random() < 0.9 else 8 * int(r.integers(33, 65))
        if chunked_only:
            Dv = 16 * ((Dv + 15) // 16)
        B = int(r.integers(1, 4))
        T = int(r.integers(64, 300) if chunked_only else r.choice([r.integers(1, 8), r.integers(8, 64),
                                                                     r.integers(64, 200)]))
        K = int(r.integers(2, 5))
        if B * T * Hv * Dk * Dv > max_work:
            continue
        out.append((B, T, Hk, Hv, Dk, Dv, K, bool(r.random() < 0.6), bool(r.random() < 0.6),
                    bool(r.random() < 0.3)))
    return out


SHAPES = sweep_shapes(20, 20261202) + sweep_shapes(12, 20261203, chunked_only=True)


@pytest.mark.parametrize("i", range(len(SHAPES)), ids=lambda i: "B%dT%dHk%dHv%dDk%dDv%dK%d-s%dc%dm%d" % SHAPES[i])
def test_layer_core_random_shapes(i):
    B, T, Hk, Hv, Dk, Dv, K, st, cs, masked = SHAPES[i]
    say("sweep", SHAPES[i])
    raw = layer_inputs(B, T, Hk, Hv, Dk, Dv, K, 900 + i, state=st, conv_state=cs)
    mask = step_mask(900 + i, B, T) if masked and T > 0 else None
    qs, ks = 1.0 / Dk, Dk ** -0.5
    y, s, cso = gpu_layer_core(raw, Hk, Hv, Dk, Dv, qs, ks, mask=mask)
    p = gpu_prep(raw, Hk, Hv, Dk, Dv, qs, ks)
    cs_ref = check_core(str(SHAPES[i]), y, s, p, raw, Hk, Hv, Dk, Dv, qs, ks, mask=mask)
    assert np.array_equal(cso, cs_ref)
    # the composition the layer core is defined as
    ri = dict(q=p["q"], k=p["k"], v=p["v"], g=p["g"], beta=p["beta"], state=raw["state"])
    chunked = H.layer_uses_chunked(B, T, Hv, Dk, Dv)
    y2, s2 = gpu_recurrent_chunked(ri, mask=mask) if chunked else gpu_recurrent(ri, mask=mask)
    assert np.array_equal(y, y2) and np.array_equal(s, s2)
