"""slimkv_decode_attn_chunk against the fp64 oracle: a chunk of Q query
tokens per sequence over a ragged cache, each token attending to the cache
and to the chunk's tokens up to itself, and the tokens stored while the raw
window has room."""

import dataclasses

import numpy as np
import pytest
import torch

import synth
from parity_util import (assert_chunk_rows, assert_parity, note, oracle_chunk, oracle_chunk_units,
                         oracle_ragged, run_gpu_chunk, run_gpu_ragged, sample_units)
from parity_util import ragged_edge_cases as edge_cases
from parity_util import ragged_workload as custom

pytestmark = pytest.mark.gpu


def check_chunk(wl, Q, *, rank_v=None, append=True, lengths=True, num_splits=0, fixed=None,
                what=""):
    inp = synth.make_layer(wl, rank_v=rank_v)
    ch = synth.make_chunk(wl, inp, Q, fixed=edge_cases(inp.num_beacons, inp.raw_window)
                          if fixed is None else fixed)
    note(f"chunk {what}: B={wl.batch} Hkv={wl.num_kv_heads} G={wl.group} Q={Q} "
         f"cap=({inp.num_beacons}, {inp.raw_window}) r=({inp.rank_k}, {inp.rank_v}) "
         f"append={append} lengths={lengths} splits={num_splits}")
    out, lse, K, V = run_gpu_chunk(inp, ch, append=append, lengths=lengths, num_splits=num_splits)
    ref, ref_lse, k_app = oracle_chunk(inp, ch, append=append, lengths=lengths)
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty), "queries without rows"
    assert np.all(out[empty] == 0.0)
    assert_parity(out, ref, wl.dtype, what, np.where(empty, 0.0, lse), np.where(empty, 0.0, ref_lse))
    # without lengths every row is live: the windows are full, nothing is stored
    written = ch if lengths else dataclasses.replace(ch, raw_len=ch.raw_len * 0 + inp.raw_window)
    assert_chunk_rows(K, V, inp.K_raw, inp.V_raw, written, k_app if append else None)
    return inp, ch, out, lse


@pytest.mark.parametrize("Q", [1, 2, 4])
def test_g4_tokens(Q, gpu_device):
    check_chunk(custom(index=140 + Q), Q, what=f"G4 Q{Q}")


def test_g1_sixteen_tokens(gpu_device):
    check_chunk(custom(B=5, Hkv=2, G=1, nb=700, w=200, r=32, index=145), 16, what="G1 Q16")


def test_g8_two_tokens(gpu_device):
    check_chunk(custom(B=6, Hkv=1, G=8, nb=500, w=100, r=128, index=146), 2, what="G8 Q2")


def test_g5_uneven_ranks(gpu_device):
    wl = custom(B=5, Hkv=3, G=5, nb=777, w=129, r=48, theta=1e6, index=147)
    check_chunk(wl, 3, rank_v=96, what="G5 Q3 r48/96")


def test_full_windows(gpu_device):
    """Windows with room for part of the chunk: the rest is attended, not stored."""
    wl = custom(B=6, Hkv=2, G=4, nb=400, w=90, index=148)
    check_chunk(wl, 4, fixed={0: (400, 90), 1: (400, 88), 2: (0, 89), 3: (10, 0), 4: (0, 0)},
                what="full windows")


def test_no_new_tokens(gpu_device):
    check_chunk(custom(index=149), 3, append=False, what="no new tokens")


def test_all_rows_no_lengths(gpu_device):
    check_chunk(custom(index=150), 2, lengths=False, what="all rows")


def test_raw_only(gpu_device):
    wl = custom(B=4, Hkv=2, G=4, nb=0, w=300, index=151)
    check_chunk(wl, 4, fixed={0: (0, 0), 1: (0, 300), 2: (0, 255)}, what="raw only")


def test_beacons_only(gpu_device):
    wl = custom(B=4, Hkv=2, G=2, nb=600, w=0, r=96, index=152)
    check_chunk(wl, 8, fixed={0: (0, 0), 1: (600, 0)}, what="beacons only")


def test_only_the_chunk(gpu_device):
    """No cache at all: each token attends to the chunk's tokens up to itself."""
    wl = custom(B=3, Hkv=2, G=4, nb=0, w=0, index=153)
    check_chunk(wl, 4, fixed={}, what="chunk only")


@pytest.mark.parametrize("splits", [1, 7, 333])
def test_grid_sizes(splits, gpu_device):
    check_chunk(custom(B=8, Hkv=2, G=4, nb=600, w=200, index=154), 4, num_splits=splits,
                what=f"grid {splits}")


def test_repeatable(gpu_device):
    wl = custom(index=155)
    _, _, a_out, a_lse = check_chunk(wl, 4, what="first")
    _, _, b_out, b_lse = check_chunk(wl, 4, what="second")
    assert np.array_equal(a_out, b_out) and np.array_equal(a_lse, b_lse)


def test_single_token_matches_ragged_call(gpu_device):
    """A chunk of one token is the ragged decode step (same oracle result;
    the two kernels sum in different orders)."""
    wl = custom(index=156)
    inp = synth.make_layer(wl)
    ch = synth.make_chunk(wl, inp, 1, fixed=edge_cases(inp.num_beacons, inp.raw_window))
    step = synth.StepInputs(ch.num_beacons, ch.raw_len, ch.k_new[:, 0].contiguous(),
                            ch.v_new[:, 0].contiguous())
    q1 = inp.q.clone()
    inp.q = ch.q[:, 0].contiguous()
    note("chunk of one vs ragged call")
    out_c, lse_c, K_c, V_c = run_gpu_chunk(inp, ch)
    out_r, lse_r, K_r, V_r = run_gpu_ragged(inp, step)
    ref, ref_lse, _ = oracle_ragged(inp, step)
    inp.q = q1
    empty = np.isneginf(ref_lse)
    for out, lse, what in ((out_c[:, 0], lse_c[:, 0], "chunk"), (out_r, lse_r, "ragged")):
        assert_parity(out, ref, "bf16", what, np.where(empty, 0.0, lse), np.where(empty, 0.0, ref_lse))
    assert np.max(np.abs(out_c[:, 0] - out_r)) < 1e-3
    assert torch.equal(K_c, K_r) and torch.equal(V_c, V_r)


# fp32 caches (the fp32 matrix-instruction kernel): the fp32 bar
@pytest.mark.parametrize("G,Q,r,rv", [(4, 4, 64, None), (1, 16, 32, None), (8, 2, 128, None),
                                      (5, 3, 48, 96)])
def test_fp32(G, Q, r, rv, gpu_device):
    wl = custom(dtype="fp32", B=5, Hkv=2, G=G, nb=300, w=70, r=r, index=160 + G * Q)
    check_chunk(wl, Q, rank_v=rv, what=f"fp32 G{G} Q{Q} r{r}")


def test_fp32_edges(gpu_device):
    """fp32: raw rows only, beacons only, windows with room for part of the
    chunk, a grid of one workgroup, no new tokens."""
    wl = custom(dtype="fp32", B=6, Hkv=2, G=4, nb=0, w=100, index=166)
    check_chunk(wl, 4, fixed={0: (0, 0), 1: (0, 100), 2: (0, 98)}, what="fp32 raw only")
    wl = custom(dtype="fp32", B=4, Hkv=2, G=2, nb=300, w=0, r=96, index=167)
    check_chunk(wl, 8, fixed={0: (0, 0), 1: (300, 0)}, what="fp32 beacons only")
    wl = custom(dtype="fp32", B=5, Hkv=2, G=4, nb=200, w=60, index=168)
    check_chunk(wl, 4, fixed={0: (200, 60), 1: (200, 58), 2: (0, 59), 3: (0, 0)}, num_splits=1,
                what="fp32 full windows, one workgroup")
    check_chunk(custom(dtype="fp32", B=4, Hkv=2, G=4, nb=250, w=50, index=169), 3, append=False,
                what="fp32 no new tokens")


@pytest.mark.parametrize("layer", [0, 6])  # ranks 48, 128
def test_c3_chunk_sampled(layer, gpu_device):
    """The 128K Llama step's shapes with 4 drafted tokens per sequence (16
    query rows per KV head): sampled units against the oracle."""
    wl = synth.get_workload("c3")
    note(f"c3 chunk layer {layer}")
    inp = synth.make_layer(wl, layer, device=gpu_device)
    ch = synth.make_chunk(wl, inp, 4, device=gpu_device, beacons=(0.5, 1.0), raw=(0.5, 1.0),
                          fixed={0: (8192, 2046), 1: (0, 0)})
    out, lse, K, V = run_gpu_chunk(inp, ch)
    units = sample_units(wl, 12, seed=layer)
    ref = oracle_chunk_units(inp, ch, units)
    G = wl.group
    got = np.stack([out[b, :, h * G:(h + 1) * G] for b, h in units])
    got_lse = np.stack([lse[b, :, h * G:(h + 1) * G] for b, h in units])
    exp = np.stack([ref[u][0] for u in units])
    exp_lse = np.stack([ref[u][1] for u in units])
    assert_parity(got, exp, wl.dtype, f"c3 chunk L{layer}", got_lse, exp_lse)
    assert_chunk_rows(K, V, inp.K_raw, inp.V_raw, ch, {u: ref[u][2] for u in units}, units=units)
    del inp, K, V
    torch.cuda.empty_cache()


def test_workspace_check_flag(gpu_device):
    """SLIMKV_FLAG_CHECK_WORKSPACE on a chunk call: counters left nonzero are
    found, cleared and reported; the result is still right."""
    import latent_decode_attention_amd as lda
    from parity_util import plant_counters
    wl = custom(B=5, Hkv=2, G=4, nb=400, w=100, index=170)
    inp = synth.make_layer(wl)
    ch = synth.make_chunk(wl, inp, 3, fixed=edge_cases(inp.num_beacons, inp.raw_window))
    note("chunk workspace check, planted counters")
    status = []
    out, lse, _, _ = run_gpu_chunk(inp, ch, num_splits=9, flags=lda.SLIMKV_FLAG_CHECK_WORKSPACE,
                                   plant=lambda ws: plant_counters(ws, wl.batch * wl.num_kv_heads),
                                   status=status)
    ref, ref_lse, _ = oracle_chunk(inp, ch)
    empty = np.isneginf(ref_lse)
    assert_parity(out, ref, wl.dtype, "chunk workspace check",
                  np.where(empty, 0.0, lse), np.where(empty, 0.0, ref_lse))
    assert status == [1]
