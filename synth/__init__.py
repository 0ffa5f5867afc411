"""Seeded synthetic inputs for SlimKV latent decode attention.

This package is shared by the tests, the benchmark and the smoke check. It
only draws random numbers and lays them out; it holds none of the attention
arithmetic (no RoPE, no projection, no softmax), so both the CPU oracle and
the HIP library can be fed from it without sharing any of the method.
"""

from .configs import RANK_SET, WORKLOADS, Workload, draw_ranks, get_workload  # noqa: F401
from .gen import (ChunkInputs, LayerInputs, PagedCache, StepInputs, alibi_slopes,  # noqa: F401
                  beacon_grid, make_chunk, make_full_kv, make_layer, make_paged, make_step, orthonormal_basis,
                  to_numpy_storage, unit_slices)
