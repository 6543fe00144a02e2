"""CPU oracle for the routed history-attention path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library."""

from . import geometry, layout, slabs
from .velox_oracle import (BLOCK, MODE_FUSED, MODE_GEOMETRY_ONLY, MODE_MODEL_ONLY,
                           attention_block, block_means, dense_attention_block, fixed_mass,
                           fused_weights, ghat, importance, importance_shared, route_row,
                           routes, sparse_attention_block)

__all__ = ["BLOCK", "MODE_FUSED", "MODE_GEOMETRY_ONLY", "MODE_MODEL_ONLY", "geometry", "layout", "slabs",
           "attention_block", "block_means", "dense_attention_block", "fixed_mass",
           "fused_weights", "ghat", "importance", "importance_shared", "route_row", "routes",
           "sparse_attention_block"]
