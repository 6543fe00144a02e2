"""Seeded synthetic inputs (shapes, router settings, q/k/v, overlaps, coverage)
for the routed history-attention path. Shared by the oracle side and the GPU
side; holds none of the method's arithmetic."""

from .workloads import (BLOCK, CHUNK_BLOCKS, RouteParams, Workload, chunk48, make_qkv,
                        sweep, tiny, trace_chunk, wan13)

__all__ = ["BLOCK", "CHUNK_BLOCKS", "RouteParams", "Workload", "chunk48", "make_qkv",
           "sweep", "tiny", "trace_chunk", "wan13"]
