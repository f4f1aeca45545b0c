"""Tile-scheduled persistent batch-1 greedy BF16 decode for MI355X (gfx950).

A host planner (C++, inside ``libtiles.so``) cuts every operator of a
Llama/Qwen3-style decoder into output-row tiles, assigns each tile to a fixed
workgroup (one per CU), groups the tiles into waves and packs the weights; one
cooperative persistent HIP kernel then executes that static schedule for up to
64 tokens per launch (Tiles page, "Tiles: Scheduling LLM Decoding as a Graph of
Tiles", intro and "What the code contains").

The C ABI is declared in ``include/tiles.h``; :mod:`.tiles` is its Python
binding (argument marshalling only).  PyTorch supplies device memory and
streams.
"""

from .configs import ModelConfig, Workload, WORKLOADS  # noqa: F401
