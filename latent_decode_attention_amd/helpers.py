"""Allocation helpers around the binding (torch device memory only)."""

from __future__ import annotations

import math

import torch

from .binding import make_problem, slimkv_problem, slimkv_workspace_bytes


def problem_from_tensors(q, U_K, C_K, K_raw, *, rope_theta: float, num_kv_heads: int,
                         scale: float | None = None, U_V=None, num_splits: int = 0,
                         flags: int = 0) -> slimkv_problem:
    """Problem struct read off the tensor shapes (C_K/U_K or K_raw may be None)."""
    B, Hq, d = q.shape
    nb = 0 if C_K is None else int(C_K.shape[2])
    rk = 0 if U_K is None else int(U_K.shape[2])
    rv = rk if U_V is None else int(U_V.shape[2])
    w = 0 if K_raw is None else int(K_raw.shape[2])
    return make_problem(batch=B, num_q_heads=Hq, num_kv_heads=num_kv_heads, num_beacons=nb,
                        rank_k=rk, rank_v=rv, raw_window=w,
                        scale=(1.0 / math.sqrt(d)) if scale is None else scale,
                        rope_theta=rope_theta, dtype=q.dtype, head_dim=d, num_splits=num_splits,
                        flags=flags)


def alloc_workspace(problem: slimkv_problem, op: int, device) -> torch.Tensor:
    """Zero-filled workspace of the size the op needs (zero on first use is
    part of the library's contract)."""
    return torch.zeros(slimkv_workspace_bytes(problem, op), dtype=torch.uint8, device=device)


def alloc_outputs(problem: slimkv_problem, device):
    out = torch.empty((problem.batch, problem.num_q_heads, problem.head_dim), dtype=torch.float32,
                      device=device)
    lse = torch.empty((problem.batch, problem.num_q_heads), dtype=torch.float32, device=device)
    return out, lse
