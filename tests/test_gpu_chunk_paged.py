"""slimkv_decode_attn_chunk_paged against the fp64 oracle, and against the
contiguous chunk call: a chunk of Q query tokens per sequence (speculative
decoding) over a cache laid out in pages drawn from shared pools.  Page ids
are a seeded permutation of each pool; rows past a sequence's live length
and pages no sequence maps are NaN, so a read of any of them would reach the
output."""

import dataclasses

import numpy as np
import pytest
import torch

import synth
from parity_util import (assert_chunk_paged_writes, assert_parity, note, oracle_chunk,
                         oracle_chunk_units, run_gpu_chunk, run_gpu_chunk_paged, sample_units)
from parity_util import ragged_edge_cases as edge_cases
from parity_util import ragged_workload as custom

pytestmark = pytest.mark.gpu


def check(wl, Q, *, page_rows=64, rank_v=None, append=True, lengths=True, num_splits=0,
          fixed=None, what=""):
    inp = synth.make_layer(wl, rank_v=rank_v)
    ch = synth.make_chunk(wl, inp, Q, fixed=edge_cases(inp.num_beacons, inp.raw_window)
                          if fixed is None else fixed)
    live = ch if lengths else dataclasses.replace(
        ch, num_beacons=torch.full_like(ch.num_beacons, inp.num_beacons),
        raw_len=torch.full_like(ch.raw_len, inp.raw_window))
    pc = synth.make_paged(inp, live, page_rows=page_rows)
    note(f"chunk paged {what}: B={wl.batch} Hkv={wl.num_kv_heads} G={wl.group} Q={Q} "
         f"cap=({inp.num_beacons}, {inp.raw_window}) r=({inp.rank_k}, {inp.rank_v}) "
         f"page_rows={page_rows} append={append} lengths={lengths} splits={num_splits}")
    out, lse, K, V = run_gpu_chunk_paged(inp, ch, pc, append=append, lengths=lengths,
                                         num_splits=num_splits)
    ref, ref_lse, k_app = oracle_chunk(inp, ch, append=append, lengths=lengths)
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty), "queries without rows"
    assert np.all(out[empty] == 0.0)
    assert_parity(out, ref, wl.dtype, what, np.where(empty, 0.0, lse), np.where(empty, 0.0, ref_lse))
    assert_chunk_paged_writes(K, V, pc, live, k_app if append else None, inp.raw_window)
    return inp, ch, pc, out, lse


@pytest.mark.parametrize("Q", [2, 4])
def test_g4_tokens(Q, gpu_device):
    check(custom(index=230 + Q), Q, what=f"G4 Q{Q}")


def test_no_new_tokens(gpu_device):
    check(custom(index=233), 3, append=False, what="no new tokens")


def test_all_rows_no_lengths(gpu_device):
    check(custom(index=234), 2, lengths=False, what="all rows")


@pytest.mark.parametrize("page_rows", [128, 1024])
def test_page_sizes_uneven_ranks(page_rows, gpu_device):
    wl = custom(B=5, Hkv=3, G=5, nb=777, w=129, r=48, theta=1e6, index=235)
    check(wl, 3, page_rows=page_rows, rank_v=96, what=f"G5 Q3 r48/96 pages of {page_rows}")


@pytest.mark.parametrize("G,Q,r", [(1, 16, 32), (8, 2, 128)])
def test_group_extremes(G, Q, r, gpu_device):
    wl = custom(B=5, Hkv=2, G=G, nb=600, w=150, r=r, index=236 + G)
    check(wl, Q, what=f"G{G} Q{Q}")


def test_tokens_cross_pages(gpu_device):
    """Chunks whose tokens' rows straddle page boundaries (pages of 64 rows),
    or run past the window (attended, not stored)."""
    wl = custom(B=6, Hkv=2, G=4, nb=300, w=200, index=245)
    check(wl, 4, fixed={0: (300, 62), 1: (10, 63), 2: (0, 127), 3: (5, 198), 4: (300, 200),
                        5: (0, 0)}, what="tokens across pages")


def test_raw_only(gpu_device):
    wl = custom(B=4, Hkv=2, G=4, nb=0, w=300, index=246)
    check(wl, 4, fixed={0: (0, 0), 1: (0, 300), 2: (0, 255)}, what="raw only")


def test_beacons_only(gpu_device):
    """No raw window: the tokens are attended, nothing is stored."""
    wl = custom(B=4, Hkv=2, G=2, nb=600, w=0, r=96, index=247)
    check(wl, 8, fixed={0: (0, 0), 1: (600, 0)}, what="beacons only")


@pytest.mark.parametrize("splits", [1, 7, 333])
def test_grid_sizes(splits, gpu_device):
    check(custom(B=8, Hkv=2, G=4, nb=600, w=200, index=248), 4, num_splits=splits,
          what=f"grid {splits}")


def test_bitwise_equal_to_contiguous(gpu_device):
    """Paging changes where rows live, not what is computed: out, lse and the
    stored rows equal the contiguous chunk call's bit for bit."""
    wl = custom(B=8, Hkv=2, G=4, nb=1000, w=300, r=64, index=249)
    inp = synth.make_layer(wl)
    ch = synth.make_chunk(wl, inp, 4, fixed=edge_cases(inp.num_beacons, inp.raw_window))
    pc = synth.make_paged(inp, ch, page_rows=64)
    note("chunk paged vs contiguous, bitwise")
    out_p, lse_p, K_p, V_p = run_gpu_chunk_paged(inp, ch, pc)
    out_c, lse_c, K_c, V_c = run_gpu_chunk(inp, ch)
    assert np.array_equal(out_p, out_c) and np.array_equal(lse_p, lse_c)
    table = pc.raw_table.numpy()
    raw_len = ch.raw_len.numpy()
    for b in range(wl.batch):
        w = int(np.clip(raw_len[b], 0, inp.raw_window))
        for u in range(4):
            if w + u >= inp.raw_window:
                break
            pid, r = int(table[b, (w + u) // 64]), (w + u) % 64
            assert torch.equal(K_p[pid, :, r], K_c[b, :, w + u])
            assert torch.equal(V_p[pid, :, r], V_c[b, :, w + u])


@pytest.mark.parametrize("page_rows", [64, 256])
def test_fp32(page_rows, gpu_device):
    wl = custom(dtype="fp32", B=5, Hkv=2, G=4, nb=400, w=150, r=48, index=250 + page_rows)
    check(wl, 3, page_rows=page_rows, what=f"fp32 pages {page_rows}")


def test_out_of_range_page_ids(gpu_device):
    """A table entry outside [0, pages) reads as a page of zeros and is never
    written: sequence 4's second beacon page is -1, and sequence 6's tokens'
    rows 126..129 fall in raw pages 1 (kept) and 2 (id -7: attended, not
    stored)."""
    wl = custom(B=8, Hkv=2, G=4, nb=600, w=200, index=250)
    inp = synth.make_layer(wl)
    fixed = edge_cases(600, 200)
    fixed.update({4: (300, 100), 5: (200, 100), 6: (100, 126)})
    ch = synth.make_chunk(wl, inp, 4, fixed=fixed)
    pc = synth.make_paged(inp, ch, page_rows=64)
    bt, rt = pc.beacon_table.clone(), pc.raw_table.clone()
    bt[4, 1] = -1
    rt[6, 2] = -7
    C_K, C_V = inp.C_K.clone(), inp.C_V.clone()
    C_K[4, :, 64:128] = 0
    C_V[4, :, 64:128] = 0
    zeroed = dataclasses.replace(inp, C_K=C_K, C_V=C_V)
    pcz = dataclasses.replace(pc, beacon_table=bt, raw_table=rt)
    note("chunk paged out-of-range ids")
    out, lse, K, V = run_gpu_chunk_paged(inp, ch, pcz)
    ref, ref_lse, k_app = oracle_chunk(zeroed, ch)
    empty = np.isneginf(ref_lse)
    assert_parity(out, ref, wl.dtype, "bad page ids", np.where(empty, 0.0, lse),
                  np.where(empty, 0.0, ref_lse))
    assert_chunk_paged_writes(K, V, pcz, ch, k_app, inp.raw_window)


@pytest.mark.parametrize("layer", [0, 6])  # ranks 48, 128
def test_c3_chunk_paged_sampled(layer, gpu_device):
    """The 128K Llama step's shapes with 4 drafted tokens per sequence, in
    pages of 64 rows: sampled units against the oracle, the whole batch
    against the contiguous call bit for bit."""
    wl = synth.get_workload("c3")
    note(f"c3 chunk paged layer {layer}")
    inp = synth.make_layer(wl, layer, device=gpu_device)
    ch = synth.make_chunk(wl, inp, 4, device=gpu_device, beacons=(0.5, 1.0), raw=(0.5, 1.0),
                          fixed={0: (8192, 2046), 1: (0, 0)})
    pc = synth.make_paged(inp, ch, page_rows=64)
    out, lse, K, V = run_gpu_chunk_paged(inp, ch, pc)
    units = sample_units(wl, 12, seed=layer)
    ref = oracle_chunk_units(inp, ch, units)
    G = wl.group
    got = np.stack([out[b, :, h * G:(h + 1) * G] for b, h in units])
    got_lse = np.stack([lse[b, :, h * G:(h + 1) * G] for b, h in units])
    exp = np.stack([ref[u][0] for u in units])
    exp_lse = np.stack([ref[u][1] for u in units])
    assert_parity(got, exp, wl.dtype, f"c3 chunk paged L{layer}", got_lse, exp_lse)
    assert_chunk_paged_writes(K, V, pc, ch.to("cpu"), {u: ref[u][2] for u in units},
                              inp.raw_window, units=units)
    del K, V, pc
    out_c, lse_c, _, _ = run_gpu_chunk(inp, ch)
    assert np.array_equal(out, out_c) and np.array_equal(lse, lse_c)
    del inp
    torch.cuda.empty_cache()
