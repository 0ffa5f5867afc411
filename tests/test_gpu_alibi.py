"""slimkv_decode_attn_alibi against the fp64 oracle: the latent decode
attention of an ALiBi backbone (no rotation; a linear distance bias added
after the scaled product, beacons on a position grid, the raw window ending
at the query)."""

import dataclasses

import numpy as np
import pytest
import torch

import synth
from parity_util import (assert_parity, gather_units, note, oracle_alibi, run_gpu, run_gpu_alibi,
                         sample_units)

pytestmark = pytest.mark.gpu


def small(dtype="bf16", B=4, Hkv=2, G=4, nb=600, w=200, r=64, context=16384, index=170):
    return dataclasses.replace(
        synth.get_workload("c2"), name="alibi", index=index, batch=B, num_q_heads=Hkv * G,
        num_kv_heads=Hkv, num_beacons=nb, raw_window=w, ranks=(r,), dtype=dtype, context=context)


def check_alibi(wl, *, ratio=16, slopes=None, rank_v=None, num_splits=0, what=""):
    inp = synth.make_layer(wl, rank_v=rank_v)
    first, stride = synth.beacon_grid(ratio)
    sl = synth.alibi_slopes(wl.num_q_heads) if slopes is None else slopes
    note(f"alibi {what}: B={wl.batch} Hkv={wl.num_kv_heads} G={wl.group} nb={inp.num_beacons} "
         f"w={inp.raw_window} r=({inp.rank_k}, {inp.rank_v}) {wl.dtype} ratio={ratio} "
         f"splits={num_splits}")
    out, lse = run_gpu_alibi(inp, sl, first, stride, num_splits=num_splits)
    ref, ref_lse = oracle_alibi(inp, sl, first, stride)
    assert_parity(out, ref, wl.dtype, what, lse, ref_lse)
    return out, lse


def test_bf16_g4(gpu_device):
    check_alibi(small(), what="bf16 G4")


def test_bf16_near_beacons(gpu_device):
    """Beacons right behind the raw window (positions 0.. at ratio 1), gentle
    slopes: beacon and raw rows both carry weight."""
    wl = small(nb=300, w=100, context=401, index=171)
    check_alibi(wl, ratio=1, slopes=np.full(8, 0.002), what="near beacons")


@pytest.mark.parametrize("G,r", [(1, 32), (5, 48), (8, 128)])
def test_groups(G, r, gpu_device):
    check_alibi(small(B=3, Hkv=2, G=G, nb=500, w=130, r=r, index=172 + G), rank_v=None,
                what=f"G{G} r{r}")


def test_uneven_ranks(gpu_device):
    check_alibi(small(B=3, Hkv=3, G=4, nb=400, w=64, r=48, index=181), rank_v=96, what="r48/96")


def test_fp32(gpu_device):
    check_alibi(small(dtype="fp32", B=3, Hkv=2, G=4, nb=300, w=45, r=32, index=182), what="fp32")


def test_raw_only(gpu_device):
    check_alibi(small(B=3, nb=0, w=257, index=183), what="raw only")


def test_beacons_only(gpu_device):
    check_alibi(small(B=3, nb=333, w=0, index=184), slopes=np.full(8, 0.001), what="beacons only")


@pytest.mark.parametrize("splits", [1, 7, 64])
def test_splits(splits, gpu_device):
    check_alibi(small(index=185), num_splits=splits, what=f"splits {splits}")


def test_zero_slopes_equal_rotary_at_position_zero(gpu_device):
    """Without bias and at position 0 the ALiBi call is the rotary call."""
    wl = small(context=1, index=186)  # the query at position 0
    inp = synth.make_layer(wl)
    out_a, lse_a = run_gpu_alibi(inp, np.zeros(8), 15, 16)
    out_r, lse_r = run_gpu(inp)
    assert np.max(np.abs(out_a - out_r)) < 2e-6 and np.max(np.abs(lse_a - lse_r)) < 2e-6


@pytest.mark.parametrize("layer", [0, 6])  # ranks 48, 128
def test_c3_alibi_sampled(layer, gpu_device):
    """The 128K Llama layer's shapes with the ALiBi paper's slopes for 32
    heads and one beacon per 16 tokens: sampled units against the oracle."""
    wl = synth.get_workload("c3")
    note(f"c3 alibi layer {layer}")
    inp = synth.make_layer(wl, layer, device=gpu_device)
    sl = synth.alibi_slopes(wl.num_q_heads)
    first, stride = synth.beacon_grid(16)
    out, lse = run_gpu_alibi(inp, sl, first, stride)
    units = sample_units(wl, 12, seed=layer)
    ref, ref_lse = oracle_alibi(inp.to("cpu"), sl, first, stride, units=units)
    got, got_lse = gather_units(out, lse, wl, units)
    exp, exp_lse = gather_units(ref, ref_lse, wl, units)
    assert_parity(got, exp, wl.dtype, f"c3 alibi L{layer}", got_lse, exp_lse)
    del inp
    torch.cuda.empty_cache()
