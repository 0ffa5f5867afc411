"""SlimKV reconstruction-free latent decode attention for AMD MI355X (gfx950).

The work happens in ``libslimkv.so`` (hand-written HIP kernels behind the C
ABI in include/slimkv.h).  This package holds its sources (csrc/), the build
script and a thin ctypes binding with the C names, plus small helpers that
allocate outputs and workspaces with torch.
"""

from .binding import (SLIMKV_BF16, SLIMKV_FLAG_CHECK_WORKSPACE,  # noqa: F401
                      SLIMKV_FLAG_DYNAMIC_TILES, SLIMKV_FP32,
                      SLIMKV_OP_FULL_KV, SLIMKV_OP_LATENT, SLIMKV_OP_LATENT_RAGGED,
                      SLIMKV_OP_RECONSTRUCT, SlimKVError, full_kv_attn, load_library,
                      make_pages, make_problem, slimkv_abi_version,
                      slimkv_chunk_workspace_bytes, slimkv_decode_attn, slimkv_decode_attn_alibi,
                      slimkv_decode_attn_chunk, slimkv_decode_attn_chunk_paged,
                      slimkv_decode_attn_noalloc, slimkv_alibi, make_alibi,
                      slimkv_decode_attn_ragged_alibi, slimkv_decode_attn_paged_alibi,
                      slimkv_decode_attn_chunk_alibi, slimkv_decode_attn_chunk_paged_alibi,
                      slimkv_decode_attn_paged, slimkv_decode_attn_ragged, slimkv_last_error,
                      slimkv_pages, slimkv_problem,
                      slimkv_reconstruct_attn, slimkv_reconstruct_rope_attn,
                      slimkv_set_kernel_events, slimkv_status_string,
                      slimkv_workspace_bytes, slimkv_workspace_status, slimkv_bench_stream_read,
                      slimkv_bench_flush)
from .helpers import alloc_outputs, alloc_workspace, problem_from_tensors  # noqa: F401
