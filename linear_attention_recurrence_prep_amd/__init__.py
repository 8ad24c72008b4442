"""Gated DeltaNet layer core for MI355X (gfx950).

The compute lives in the HIP library ``libgdn.so`` (built from ``csrc/``),
reached through its C ABI (``include/gdn.h``).  ``binding`` marshals torch
tensors to that ABI; ``inputs`` draws seeded synthetic inputs.  The library
is loaded on first use; if it has not been built, that first call raises.
"""
from .binding import (  # noqa: F401
    Bound, GdnError, bind, gated_rmsnorm, layer_core, layer_core_gated, layer_core_workspace_bytes, lib, prep,
    recurrent, recurrent_chunked, recurrent_chunked_per_key, recurrent_chunked_per_key_workspace_bytes,
    recurrent_chunked_workspace_bytes, recurrent_per_key, recurrent_snapshots,
)
