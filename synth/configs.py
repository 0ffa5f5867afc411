"""Workload shapes for latent decode attention, as plain data.

The shapes follow the two backbones the SlimKV evaluation uses (page
"Can SlimKV compress KV cache jointly across tokens and features",
section "LongBench gains concentrate at high compression": Llama-3.1-8B and
Qwen2.5-14B) and the 128K / 16x and 32x decode-latency setting of section
"Speedups are real, but memory is set by the ratio".

Each workload is a list of layers; a layer is one independent call of the
attention entry point (ranks can differ per layer, section "Beacon states
carry implicit position cues": rank is allocated per layer).

Conventions that the pages leave open and that these shapes fix:
  * the decode query sits at the last context position, q_pos = T - 1;
  * the raw window holds positions T-W .. T-1 and is already RoPE'd;
  * beacons carry no position (their keys are K-RoPE-free);
  * scale = 1/sqrt(head_dim) for beacon and raw scores alike.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

RANK_SET = (32, 48, 64, 96, 128)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic decode-attention workload (all layers share the shape)."""

    name: str
    index: int  # stable id mixed into the seeds
    layers: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    context: int  # T, tokens of history the cache stands for
    num_beacons: int  # N_b (0 = no beacon memory, i.e. full KV)
    ranks: tuple  # per-layer rank, r_K = r_V
    raw_window: int  # W
    rope_theta: float
    dtype: str  # "fp32" or "bf16"
    sigma: float  # std of every generated Gaussian except the bases U

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def q_pos(self) -> int:
        return self.context - 1

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    def layer_bytes(self, layer: int) -> int:
        """Cache bytes one layer's call must stream (latent + raw rows)."""
        r = self.ranks[layer]
        per_unit = self.num_beacons * 2 * r + 2 * self.raw_window * self.head_dim
        return self.batch * self.num_kv_heads * per_unit * self.elem_bytes

    def step_bytes(self) -> int:
        return sum(self.layer_bytes(layer) for layer in range(self.layers))


def draw_ranks(layers: int, mean_rank: int, seed: int, rank_set=RANK_SET) -> tuple:
    """Per-layer ranks drawn i.i.d. from ``rank_set``, then nudged so that
    their sum is exactly ``layers * mean_rank``.

    A seeded stand-in for the paper's layer-adaptive allocation (whose
    formula is not on the pages): each nudge moves one layer, visited in a
    seeded order, one step along ``rank_set`` toward the target without
    overshooting it.  When no single step fits, one layer at 96 drops to 64
    and one at 32 rises to 48 (net -16), which always unblocks the walk.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, layers, mean_rank])))
    steps = list(rank_set)
    ranks = [int(x) for x in rng.choice(steps, size=layers)]
    target = layers * mean_rank
    order = [int(i) for i in rng.permutation(layers)]
    for _ in range(100 * layers):
        total = sum(ranks)
        if total == target:
            return tuple(ranks)
        moved = False
        for i in order:
            pos = steps.index(ranks[i])
            nxt = pos + 1 if total < target else pos - 1
            if 0 <= nxt < len(steps):
                delta = steps[nxt] - ranks[i]
                if abs(total + delta - target) < abs(total - target) and (
                    (total < target and total + delta <= target)
                    or (total > target and total + delta >= target)
                ):
                    ranks[i] = steps[nxt]
                    moved = True
                    break
        if not moved:
            hi = [i for i in order if ranks[i] == 96]
            lo = [i for i in order if ranks[i] == 32]
            if not hi or not lo:
                raise RuntimeError("rank draw cannot reach its target")
            ranks[hi[0]] = 64
            ranks[lo[0]] = 48
        order = order[1:] + order[:1]
    raise RuntimeError("rank draw did not converge")


def _c1():
    return Workload("c1_fp32_4k_8x", 1, layers=1, batch=1, num_q_heads=4, num_kv_heads=1,
                    head_dim=128, context=4096, num_beacons=512, ranks=(32,), raw_window=128,
                    rope_theta=500000.0, dtype="fp32", sigma=1.0)


def _c2():
    return Workload("c2_llama_layer_32k_8x", 2, layers=1, batch=8, num_q_heads=32, num_kv_heads=8,
                    head_dim=128, context=32768, num_beacons=4096, ranks=(64,), raw_window=1024,
                    rope_theta=500000.0, dtype="bf16", sigma=0.5)


def _c3():
    return Workload("c3_llama8b_128k_16x_step", 3, layers=32, batch=16, num_q_heads=32,
                    num_kv_heads=8, head_dim=128, context=131072, num_beacons=8192,
                    ranks=draw_ranks(32, 64, seed=3), raw_window=2048, rope_theta=500000.0,
                    dtype="bf16", sigma=1.0)


def _c4():
    return Workload("c4_qwen14b_128k_32x_step", 4, layers=48, batch=32, num_q_heads=40,
                    num_kv_heads=8, head_dim=128, context=131072, num_beacons=4096,
                    ranks=draw_ranks(48, 64, seed=4), raw_window=1024, rope_theta=1000000.0,
                    dtype="bf16", sigma=1.0)


def _c5(ratio: int):
    return Workload(f"c5_llama_layer_128k_{ratio}x", 5, layers=1, batch=16, num_q_heads=32,
                    num_kv_heads=8, head_dim=128, context=131072, num_beacons=131072 // ratio,
                    ranks=(64,), raw_window=2048, rope_theta=500000.0, dtype="bf16", sigma=1.0)


def _c5_full():
    return Workload("c5_llama_layer_128k_full_kv", 5, layers=1, batch=16, num_q_heads=32,
                    num_kv_heads=8, head_dim=128, context=131072, num_beacons=0, ranks=(64,),
                    raw_window=131072, rope_theta=500000.0, dtype="bf16", sigma=1.0)


WORKLOADS = {
    "c1": _c1(),
    "c2": _c2(),
    "c3": _c3(),
    "c4": _c4(),
    "c5_4x": _c5(4),
    "c5_8x": _c5(8),
    "c5_16x": _c5(16),
    "c5_32x": _c5(32),
    "c5_full": _c5_full(),
}


def get_workload(key: str) -> Workload:
    return WORKLOADS[key]
