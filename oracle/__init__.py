"""fp64 CPU oracle for the attention hot path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product package.
"""
from .attn_oracle import (  # noqa: F401
    TILE_EMPTY, TILE_FULL, TILE_PARTIAL, additive_mask, allowed_mask,
    allowed_pairs, attn_ref, decode_ref, decode_split_ref, split_bounds,
    tile_plan_ref,
)
