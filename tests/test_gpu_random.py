"""Seeded random shapes for every entry point, against the fp64 oracle.

The other GPU tests pick their shapes by hand; here a fixed-seed generator
draws them -- batch, heads, group size, key and value ranks (any multiple of
16 up to d), capacities, grid sizes, per-sequence lengths with the edge
cases mixed in, page sizes, chunk sizes, ALiBi grids -- so that
combinations nobody picked are compared element by element too.  Each case
is named by its parameters in the test id."""

import dataclasses

import numpy as np
import pytest
import torch

import latent_decode_attention_amd as lda
import synth
from parity_util import (RECON_LSE_TOL, assert_chunk_rows, assert_new_rows, assert_paged_writes,
                         assert_parity, note, oracle_alibi, oracle_chunk, oracle_layer,
                         oracle_ragged, run_gpu, run_gpu_alibi, run_gpu_chunk, run_gpu_paged,
                         run_gpu_ragged)

pytestmark = pytest.mark.gpu

RANKS = tuple(range(16, 129, 16))

# The kernels score with a hi + lo bf16 split of the fp32 query and
# accumulate in fp32, so on bf16 caches they land within ~1e-5 of the fp64
# oracle (worst measured over these cases: 4.3e-6 relative L2), far inside
# the 5e-3 stated for bf16 caches.  This tighter bound catches a lost
# precision step (a dropped lo term costs ~1e-3) that the stated one would
# let through; the reconstruct path, which rounds its rebuilt keys to bf16,
# is held to the stated bar only.
DESIGN_REL_L2 = 1e-4


def assert_design_accuracy(out, ref, dtype, what):
    if dtype == "bf16":
        rel = float(np.linalg.norm(out - ref) / max(np.linalg.norm(ref), 1e-300))
        assert rel <= DESIGN_REL_L2, f"{what}: rel-L2 {rel:.3e} above the kernels' design accuracy"


def workload(dtype, B, Hkv, G, nb, w, rk, theta, context, index):
    return dataclasses.replace(
        synth.get_workload("c2"), name="random", index=index, batch=B, num_q_heads=Hkv * G,
        num_kv_heads=Hkv, num_beacons=nb, raw_window=w, ranks=(rk,), dtype=dtype, sigma=1.0,
        rope_theta=theta, context=context)


def draw_shape(rng, *, bf16_only=False, max_group=8):
    dtype = "bf16" if bf16_only or rng.random() < 0.7 else "fp32"
    B = int(rng.integers(1, 7))
    Hkv = int(rng.integers(1, 4))
    G = int(rng.integers(1, max_group + 1))
    nb = int(rng.choice([0, 1, 15, 16, 17, 63, 64, 65, int(rng.integers(2, 1500))]))
    w = int(rng.choice([0, 1, 16, 31, int(rng.integers(2, 400))]))
    if nb + w == 0:
        w = 1
    rk, rv = int(rng.choice(RANKS)), int(rng.choice(RANKS))
    theta = float(rng.choice([5e5, 1e6, 1e4]))
    return dict(dtype=dtype, B=B, Hkv=Hkv, G=G, nb=nb, w=w, rk=rk, rv=rv, theta=theta)


def case_id(c):
    return "-".join(f"{k}{v}" for k, v in c.items() if k != "seed")


def cases(seed, n, **kw):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        c = draw_shape(rng, **kw)
        c["seed"] = seed * 100 + i
        out.append(c)
    return out


def layer(c, index, context=None):
    ctx = context if context is not None else max(4096, c["nb"] * 16 + c["w"] + 1)
    wl = workload(c["dtype"], c["B"], c["Hkv"], c["G"], c["nb"], c["w"], c["rk"], c["theta"], ctx,
                  index)
    return wl, synth.make_layer(wl, base_seed=c["seed"], rank_v=c["rv"])


def draw_lengths(rng, B, nb, w):
    """Per-sequence (beacons, raw) with the edge cases mixed in: none, full,
    beyond the capacity, one row, anything in between."""
    fixed = {}
    for b in range(B):
        kind = int(rng.integers(0, 5))
        if kind == 0:
            fixed[b] = (0, 0)
        elif kind == 1:
            fixed[b] = (nb, w)
        elif kind == 2:
            fixed[b] = (nb + int(rng.integers(1, 9)), -int(rng.integers(1, 5)))
        elif kind == 3:
            fixed[b] = (min(1, nb), min(1, w))
        else:
            fixed[b] = (int(rng.integers(0, nb + 1)), int(rng.integers(0, w + 1)))
    return fixed


UNIFORM = cases(1, 12)


@pytest.mark.parametrize("c", UNIFORM, ids=case_id)
def test_latent(c, gpu_device):
    wl, inp = layer(c, 200)
    splits = int(np.random.default_rng(c["seed"]).choice([0, 1, 2, 5, 64]))
    note(f"random latent {case_id(c)} splits={splits}")
    out, lse = run_gpu(inp, lda.SLIMKV_OP_LATENT, num_splits=splits)
    ref, ref_lse = oracle_layer(inp)
    assert_parity(out, ref, c["dtype"], f"random latent {case_id(c)}", lse, ref_lse)
    assert_design_accuracy(out, ref, c["dtype"], "latent")


@pytest.mark.parametrize("c", cases(2, 6), ids=case_id)
def test_reconstruct(c, gpu_device):
    wl, inp = layer(c, 201)
    note(f"random reconstruct {case_id(c)}")
    out, lse = run_gpu(inp, lda.SLIMKV_OP_RECONSTRUCT)
    ref, ref_lse = oracle_layer(inp)
    assert_parity(out, ref, c["dtype"], f"random reconstruct {case_id(c)}", lse, ref_lse,
                  lse_tol=RECON_LSE_TOL[c["dtype"]])


@pytest.mark.parametrize("c", cases(3, 12), ids=case_id)
def test_ragged(c, gpu_device):
    rng = np.random.default_rng(c["seed"])
    wl, inp = layer(c, 202)
    step = synth.make_step(wl, inp, base_seed=c["seed"],
                           fixed=draw_lengths(rng, c["B"], c["nb"], c["w"]))
    append = bool(rng.random() < 0.75)
    splits = int(rng.choice([0, 1, 3, 37, 512]))
    note(f"random ragged {case_id(c)} append={append} splits={splits}")
    out, lse, K, V = run_gpu_ragged(inp, step, append=append, num_splits=splits)
    ref, ref_lse, k_app = oracle_ragged(inp, step, append=append)
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty), "sequences without rows"
    assert np.all(out[empty] == 0.0)
    assert_parity(out, ref, c["dtype"], f"random ragged {case_id(c)}", np.where(empty, 0.0, lse),
                  np.where(empty, 0.0, ref_lse))
    assert_design_accuracy(out, ref, c["dtype"], "ragged")
    if append:
        assert_new_rows(K, V, inp.K_raw, inp.V_raw, step, k_app)
    else:
        assert torch.equal(K, inp.K_raw) and torch.equal(V, inp.V_raw)


@pytest.mark.parametrize("c", cases(4, 8), ids=case_id)
def test_paged(c, gpu_device):
    rng = np.random.default_rng(c["seed"])
    wl, inp = layer(c, 203)
    step = synth.make_step(wl, inp, base_seed=c["seed"],
                           fixed=draw_lengths(rng, c["B"], c["nb"], c["w"]))
    page_rows = int(rng.choice([64, 128, 256, 1024]))
    pc = synth.make_paged(inp, step, page_rows=page_rows, base_seed=c["seed"])
    note(f"random paged {case_id(c)} page_rows={page_rows}")
    out, lse, K, V = run_gpu_paged(inp, step, pc)
    ref, ref_lse, k_app = oracle_ragged(inp, step, append=True)
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty), "sequences without rows"
    assert_parity(out, ref, c["dtype"], f"random paged {case_id(c)}", np.where(empty, 0.0, lse),
                  np.where(empty, 0.0, ref_lse))
    assert_design_accuracy(out, ref, c["dtype"], "paged")
    assert_paged_writes(K, V, pc, step, k_app, inp.raw_window)


@pytest.mark.parametrize("c", cases(5, 10, bf16_only=True), ids=case_id)
def test_chunk(c, gpu_device):
    rng = np.random.default_rng(c["seed"])
    wl, inp = layer(c, 204)
    Q = int(rng.integers(1, 16 // c["G"] + 1))
    ch = synth.make_chunk(wl, inp, Q, base_seed=c["seed"],
                          fixed=draw_lengths(rng, c["B"], c["nb"], c["w"]))
    append = bool(rng.random() < 0.75)
    note(f"random chunk {case_id(c)} Q={Q} append={append}")
    out, lse, K, V = run_gpu_chunk(inp, ch, append=append)
    ref, ref_lse, k_app = oracle_chunk(inp, ch, append=append)
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty), "query rows without keys"
    assert_parity(out, ref, c["dtype"], f"random chunk {case_id(c)} Q={Q}",
                  np.where(empty, 0.0, lse), np.where(empty, 0.0, ref_lse))
    assert_design_accuracy(out, ref, c["dtype"], "chunk")
    assert_chunk_rows(K, V, inp.K_raw, inp.V_raw, ch, k_app if append else None)


@pytest.mark.parametrize("c", cases(6, 8), ids=case_id)
def test_alibi(c, gpu_device):
    rng = np.random.default_rng(c["seed"])
    ratio = int(rng.choice([1, 4, 16]))
    wl, inp = layer(c, 205, context=c["nb"] * ratio + c["w"] + int(rng.integers(1, 50)))
    first, stride = synth.beacon_grid(ratio)
    slopes = synth.alibi_slopes(wl.num_q_heads)
    if rng.random() < 0.5:
        slopes = slopes * float(rng.choice([0.01, 0.1]))
    splits = int(rng.choice([0, 1, 7]))
    note(f"random alibi {case_id(c)} ratio={ratio} splits={splits}")
    out, lse = run_gpu_alibi(inp, slopes, first, stride, num_splits=splits)
    ref, ref_lse = oracle_alibi(inp, slopes, first, stride)
    assert_parity(out, ref, c["dtype"], f"random alibi {case_id(c)}", lse, ref_lse)
    assert_design_accuracy(out, ref, c["dtype"], "alibi")
