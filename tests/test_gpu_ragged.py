"""slimkv_decode_attn_ragged against the fp64 oracle: ragged batches in
capacity-sized arrays, and the decode step's new token (attended as a rotated
raw row, and stored when the window has room)."""

import numpy as np
import pytest
import torch

import synth
from parity_util import assert_new_rows, assert_parity, gather_units, note, oracle_layer
from parity_util import oracle_ragged, oracle_ragged_units, run_gpu, run_gpu_ragged, sample_units
from parity_util import ragged_edge_cases as edge_cases
from parity_util import ragged_workload as custom

pytestmark = pytest.mark.gpu


def check_ragged(wl, *, rank_v=None, append=True, lengths=True, num_splits=0, fixed=None,
                 what=""):
    inp = synth.make_layer(wl, rank_v=rank_v)
    step = synth.make_step(wl, inp, fixed=edge_cases(inp.num_beacons, inp.raw_window)
                           if fixed is None else fixed)
    note(f"ragged {what}: B={wl.batch} Hkv={wl.num_kv_heads} G={wl.group} "
         f"cap=({inp.num_beacons}, {inp.raw_window}) r=({inp.rank_k}, {inp.rank_v}) {wl.dtype} "
         f"append={append} lengths={lengths} splits={num_splits}")
    out, lse, K, V = run_gpu_ragged(inp, step, append=append, lengths=lengths,
                                    num_splits=num_splits)
    ref, ref_lse, k_app = oracle_ragged(inp, step, append=append, lengths=lengths)
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty), "sequences without rows"
    assert np.all(out[empty] == 0.0)
    assert_parity(out, ref, wl.dtype, what, np.where(empty, 0.0, lse), np.where(empty, 0.0, ref_lse))
    if append:
        assert_new_rows(K, V, inp.K_raw, inp.V_raw, step, k_app)
    else:
        assert torch.equal(K, inp.K_raw) and torch.equal(V, inp.V_raw)
    return out, lse


def test_bf16_append(gpu_device):
    check_ragged(custom(), what="bf16 G4 append")


def test_bf16_lengths_only(gpu_device):
    check_ragged(custom(), append=False, what="bf16 G4 no new token")


def test_bf16_g5_uneven_ranks(gpu_device):
    wl = custom(B=5, Hkv=3, G=5, nb=777, w=129, r=48, theta=1e6, index=96)
    check_ragged(wl, rank_v=96, what="bf16 G5 r48/96")


@pytest.mark.parametrize("G,r", [(1, 32), (8, 128)])
def test_bf16_group_extremes(G, r, gpu_device):
    check_ragged(custom(B=6, Hkv=1, G=G, nb=500, w=70, r=r, index=97 + G), what=f"bf16 G{G}")


def test_fp32(gpu_device):
    wl = custom(dtype="fp32", B=6, Hkv=2, G=5, nb=300, w=45, r=32, index=99)
    check_ragged(wl, what="fp32 G5")


def test_fp32_no_beacons(gpu_device):
    wl = custom(dtype="fp32", B=4, Hkv=2, G=4, nb=0, w=64, r=32, index=100)
    check_ragged(wl, fixed={0: (0, 0), 1: (0, 64), 2: (0, 63)}, what="fp32 raw only")


def test_only_new_token(gpu_device):
    """No cache capacity at all: each sequence attends only to its new token
    (nothing can be stored)."""
    wl = custom(B=4, Hkv=2, G=4, nb=0, w=0, index=101)
    check_ragged(wl, fixed={}, what="new token only")
    check_ragged(wl, fixed={}, append=False, what="nothing at all")


@pytest.mark.parametrize("splits", [1, 2, 7, 15, 16, 17, 64, 333])
def test_grid_sizes(splits, gpu_device):
    """Shares that cut units anywhere (down to one workgroup for the batch);
    16 slots for the 16 units is the largest grid scheduled one piece per
    unit without a search, 17 the smallest searched."""
    check_ragged(custom(B=8, Hkv=2, G=4, nb=600, w=200, index=102), num_splits=splits,
                 what=f"grid {splits}")


def test_repeatable(gpu_device):
    wl = custom(index=103)
    a = check_ragged(wl, what="first")
    b = check_ragged(wl, what="second")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_full_lengths_match_plain_call(gpu_device):
    """No lengths and no new token: the plain entry point's problem."""
    inp = synth.make_layer(custom(B=4, index=104))
    step = synth.make_step(inp.workload, inp)
    out, lse, _, _ = run_gpu_ragged(inp, step, append=False, lengths=False)
    ref, ref_lse = oracle_layer(inp)
    assert_parity(out, ref, "bf16", "ragged, full lengths", lse, ref_lse)
    plain, plain_lse = run_gpu(inp)
    assert np.max(np.abs(plain - out)) < 1e-3


@pytest.mark.parametrize("layer", [0, 6])  # ranks 48, 128
def test_c3_ragged_sampled(layer, gpu_device):
    """The 128K Llama step's shapes: beacons live from half to all of 8192,
    raw rows from half to all of 2048 minus one, and the new token."""
    wl = synth.get_workload("c3")
    note(f"c3 ragged layer {layer}")
    inp = synth.make_layer(wl, layer, device=gpu_device)
    step = synth.make_step(wl, inp, device=gpu_device, beacons=(0.5, 1.0), raw=(0.5, 1.0),
                           fixed={0: (8192, 2047), 1: (0, 0)})
    out, lse, K, V = run_gpu_ragged(inp, step)
    units = sample_units(wl, 12, seed=layer)
    ref = oracle_ragged_units(inp, step, units)
    got, got_lse = gather_units(out, lse, wl, units)
    exp = np.stack([ref[u][0] for u in units])
    exp_lse = np.stack([ref[u][1] for u in units])
    assert_parity(got, exp, wl.dtype, f"c3 ragged L{layer}", got_lse, exp_lse)
    k_app = {u: ref[u][2] for u in units}
    assert_new_rows(K, V, inp.K_raw, inp.V_raw, step, k_app, units=units)
    del inp, K, V
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,splits", [(200, 0), (200, 150), (1024, 0)])
def test_large_batches(B, splits, gpu_device):
    """Batches past 64 sequences (each schedule lane takes several), with
    more slots than units and with fewer (one piece per unit)."""
    wl = custom(B=B, Hkv=1, G=4, nb=64, w=40, r=32, index=105 + B % 7)
    fixed = {0: (0, 0), 1: (64, 40), B - 1: (70, -3), B // 2: (1, 0)}
    check_ragged(wl, num_splits=splits, fixed=fixed, what=f"B={B} splits={splits}")


@pytest.mark.parametrize("B", [64, 65])
def test_schedule_batch_boundary(B, gpu_device):
    """64 sequences: the largest batch whose share search runs on all four
    waves of a workgroup (one sequence per lane); 65: the single-wave
    schedule with several sequences per lane."""
    wl = custom(B=B, Hkv=2, G=4, nb=96, w=40, r=32, index=107 + B % 5)
    fixed = {0: (0, 0), 1: (96, 40), B - 1: (50, 3), B // 2: (1, 0)}
    check_ragged(wl, fixed=fixed, what=f"B={B}")


def test_schedule_wide_share_range(gpu_device):
    """One sequence of 129 tiles (8192 beacons in 64-row tiles, and a raw
    tile) among fifteen of two, in 17 workgroup slots for 16 units: the
    candidate shares run from 10 to 129, more than the 64 a wave tests at
    once, so the schedule takes the single-wave bisection."""
    wl = custom(B=16, Hkv=1, G=4, nb=8192, w=16, r=32, index=110)
    fixed = {i: ((8192, 4) if i == 0 else (8, 4)) for i in range(16)}
    check_ragged(wl, fixed=fixed, num_splits=17, what="wide share range")


@pytest.mark.parametrize("planted", [False, True])
def test_workspace_check_flag(planted, gpu_device):
    """SLIMKV_FLAG_CHECK_WORKSPACE on a ragged call: counters left nonzero (as
    by an interrupted call) are found, cleared and reported, and the result
    is still right; a clean workspace reports nothing."""
    import latent_decode_attention_amd as lda
    from parity_util import plant_counters
    wl = custom(B=6, Hkv=2, G=4, nb=500, w=120, index=180 + planted)
    inp = synth.make_layer(wl)
    step = synth.make_step(wl, inp, fixed=edge_cases(inp.num_beacons, inp.raw_window))
    note(f"ragged workspace check, planted={planted}")
    status = []
    out, lse, _, _ = run_gpu_ragged(inp, step, num_splits=7, flags=lda.SLIMKV_FLAG_CHECK_WORKSPACE,
                                    plant=(lambda ws: plant_counters(ws, wl.batch * wl.num_kv_heads))
                                    if planted else None, status=status)
    ref, ref_lse, _ = oracle_ragged(inp, step)
    empty = np.isneginf(ref_lse)
    assert_parity(out, ref, wl.dtype, f"workspace check planted={planted}",
                  np.where(empty, 0.0, lse), np.where(empty, 0.0, ref_lse))
    assert status == [1 if planted else 0]
