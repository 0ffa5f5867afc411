"""slimkv_decode_attn_paged against the fp64 oracle, and against the
contiguous ragged call: the same step over a cache laid out in pages drawn
from shared pools through per-sequence page tables.  Page ids are a seeded
permutation of each pool; rows past a sequence's live length and pages no
sequence maps are NaN, so a read of any of them would reach the output."""

import dataclasses

import numpy as np
import pytest
import torch

import synth
from parity_util import (assert_paged_writes, assert_parity, gather_units, note, oracle_ragged,
                         oracle_ragged_units, run_gpu_paged, run_gpu_ragged, sample_units)
from parity_util import ragged_edge_cases as edge_cases
from parity_util import ragged_workload as custom

pytestmark = pytest.mark.gpu


def full_lengths(inp, step):
    """step with every row of the capacity live (what a call without
    lengths reads)."""
    B = step.num_beacons.shape[0]
    return dataclasses.replace(
        step, num_beacons=torch.full((B,), inp.num_beacons, dtype=torch.int32),
        raw_len=torch.full((B,), inp.raw_window, dtype=torch.int32))


def check_oracle(inp, step, out, lse, *, append, lengths, what):
    ref, ref_lse, k_app = oracle_ragged(inp, step, append=append, lengths=lengths)
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty), "sequences without rows"
    assert np.all(out[empty] == 0.0)
    assert_parity(out, ref, inp.workload.dtype, what, np.where(empty, 0.0, lse),
                  np.where(empty, 0.0, ref_lse))
    return k_app


def check_paged(wl, *, page_rows=64, rank_v=None, append=True, lengths=True, num_splits=0,
                fixed=None, what=""):
    inp = synth.make_layer(wl, rank_v=rank_v)
    step = synth.make_step(wl, inp, fixed=edge_cases(inp.num_beacons, inp.raw_window)
                           if fixed is None else fixed)
    pc = synth.make_paged(inp, step if lengths else full_lengths(inp, step), page_rows=page_rows)
    note(f"paged {what}: B={wl.batch} Hkv={wl.num_kv_heads} G={wl.group} "
         f"cap=({inp.num_beacons}, {inp.raw_window}) r=({inp.rank_k}, {inp.rank_v}) {wl.dtype} "
         f"page_rows={page_rows} pools=({pc.beacon_pages}, {pc.raw_pages}) append={append} "
         f"lengths={lengths} splits={num_splits}")
    out, lse, K, V = run_gpu_paged(inp, step, pc, append=append, lengths=lengths,
                                   num_splits=num_splits)
    k_app = check_oracle(inp, step, out, lse, append=append, lengths=lengths, what=what)
    assert_paged_writes(K, V, pc, step, k_app if append else None, inp.raw_window)
    return inp, step, pc, out, lse


def test_bf16_append(gpu_device):
    check_paged(custom(index=110), what="bf16 G4 append")


def test_bf16_no_new_token(gpu_device):
    check_paged(custom(index=111), append=False, what="bf16 G4 no new token")


def test_bf16_all_rows(gpu_device):
    check_paged(custom(index=112), append=False, lengths=False, what="bf16 G4 all rows")


@pytest.mark.parametrize("page_rows", [128, 1024])
def test_page_sizes_uneven_ranks(page_rows, gpu_device):
    wl = custom(B=5, Hkv=3, G=5, nb=777, w=129, r=48, theta=1e6, index=113)
    check_paged(wl, rank_v=96, page_rows=page_rows, what=f"bf16 G5 r48/96 pages of {page_rows}")


@pytest.mark.parametrize("G,r", [(1, 32), (8, 128)])
def test_group_extremes(G, r, gpu_device):
    check_paged(custom(B=6, Hkv=1, G=G, nb=500, w=70, r=r, index=114 + G), what=f"bf16 G{G}")


def test_fp32(gpu_device):
    wl = custom(dtype="fp32", B=6, Hkv=2, G=5, nb=300, w=45, r=32, index=124)
    check_paged(wl, what="fp32 G5")


def test_raw_only(gpu_device):
    wl = custom(dtype="fp32", B=4, Hkv=2, G=4, nb=0, w=200, r=32, index=125)
    check_paged(wl, fixed={0: (0, 0), 1: (0, 200), 2: (0, 128)}, what="fp32 raw only")


def test_beacons_only(gpu_device):
    """No raw window: the new token is attended, nothing is stored."""
    wl = custom(B=4, Hkv=2, G=4, nb=300, w=0, index=126)
    check_paged(wl, fixed={0: (0, 0), 1: (300, 0)}, what="beacons only")


@pytest.mark.parametrize("splits", [1, 7, 333])
def test_grid_sizes(splits, gpu_device):
    check_paged(custom(B=8, Hkv=2, G=4, nb=600, w=200, index=127), num_splits=splits,
                what=f"grid {splits}")


def test_bitwise_equal_to_contiguous(gpu_device):
    """Paging changes where rows live, not what is computed: out, lse and the
    stored rows equal the contiguous ragged call's bit for bit."""
    wl = custom(B=8, Hkv=2, G=4, nb=1000, w=300, r=64, index=128)
    inp = synth.make_layer(wl)
    step = synth.make_step(wl, inp, fixed=edge_cases(inp.num_beacons, inp.raw_window))
    pc = synth.make_paged(inp, step, page_rows=64)
    note("paged vs contiguous, bitwise")
    out_p, lse_p, K_p, V_p = run_gpu_paged(inp, step, pc)
    out_c, lse_c, K_c, V_c = run_gpu_ragged(inp, step)
    assert np.array_equal(out_p, out_c) and np.array_equal(lse_p, lse_c)
    table = pc.raw_table.numpy()
    raw_len = step.raw_len.numpy()
    for b in range(wl.batch):
        w = int(np.clip(raw_len[b], 0, inp.raw_window))
        if w < inp.raw_window:
            pid, r = int(table[b, w // 64]), w % 64
            assert torch.equal(K_p[pid, :, r], K_c[b, :, w])
            assert torch.equal(V_p[pid, :, r], V_c[b, :, w])


def test_shared_prefix(gpu_device):
    """Sequences 4 and 5 read sequence 6's first two beacon pages (a common
    prefix): their logical rows are then that sequence's."""
    wl = custom(B=8, Hkv=2, G=4, nb=600, w=200, index=129)
    inp = synth.make_layer(wl)
    step = synth.make_step(wl, inp, beacons=(0.5, 1.0), fixed=edge_cases(600, 200))
    pc = synth.make_paged(inp, step, page_rows=64)
    bt = pc.beacon_table.clone()
    C_K, C_V = inp.C_K.clone(), inp.C_V.clone()
    for b in (4, 5):
        bt[b, :2] = bt[6, :2]
        C_K[b, :, :128] = inp.C_K[6, :, :128]
        C_V[b, :, :128] = inp.C_V[6, :, :128]
    shared = dataclasses.replace(inp, C_K=C_K, C_V=C_V)
    note("paged shared prefix")
    out, lse, K, V = run_gpu_paged(inp, step, pc, beacon_table=bt)
    k_app = check_oracle(shared, step, out, lse, append=True, lengths=True, what="shared prefix")
    assert_paged_writes(K, V, pc, step, k_app, inp.raw_window)


def test_out_of_range_page_ids(gpu_device):
    """A table entry outside [0, pages) reads as a page of zeros and is never
    written: sequence 4's second beacon page is -1, sequence 5's first raw
    page is past the pool, sequence 6's new row falls in a page with id -7
    (attended, not stored)."""
    wl = custom(B=8, Hkv=2, G=4, nb=600, w=200, index=130)
    inp = synth.make_layer(wl)
    fixed = edge_cases(600, 200)
    fixed.update({4: (300, 100), 5: (200, 100), 6: (100, 128)})
    step = synth.make_step(wl, inp, fixed=fixed)
    pc = synth.make_paged(inp, step, page_rows=64)
    bt, rt = pc.beacon_table.clone(), pc.raw_table.clone()
    bt[4, 1] = -1
    rt[5, 0] = pc.raw_pages + 5
    rt[6, 2] = -7
    C_K, C_V, K_raw, V_raw = (x.clone() for x in (inp.C_K, inp.C_V, inp.K_raw, inp.V_raw))
    C_K[4, :, 64:128] = 0
    C_V[4, :, 64:128] = 0
    K_raw[5, :, 0:64] = 0
    V_raw[5, :, 0:64] = 0
    zeroed = dataclasses.replace(inp, C_K=C_K, C_V=C_V, K_raw=K_raw, V_raw=V_raw)
    note("paged out-of-range ids")
    out, lse, K, V = run_gpu_paged(inp, step, pc, beacon_table=bt, raw_table=rt)
    k_app = check_oracle(zeroed, step, out, lse, append=True, lengths=True, what="bad page ids")
    assert_paged_writes(K, V, pc, step, k_app, inp.raw_window, raw_table=rt)


@pytest.mark.parametrize("layer", [0, 6])  # ranks 48, 128
def test_c3_paged_sampled(layer, gpu_device):
    """The 128K Llama step's shapes in pages of 64 rows: beacons live from
    half to all of 8192, raw rows from half to all of 2048 minus one, and
    the new token; sampled units against the oracle, the whole batch
    against the contiguous call bit for bit."""
    wl = synth.get_workload("c3")
    note(f"c3 paged layer {layer}")
    inp = synth.make_layer(wl, layer, device=gpu_device)
    step = synth.make_step(wl, inp, device=gpu_device, beacons=(0.5, 1.0), raw=(0.5, 1.0),
                           fixed={0: (8192, 2047), 1: (0, 0)})
    pc = synth.make_paged(inp, step, page_rows=64)
    out, lse, K, V = run_gpu_paged(inp, step, pc)
    units = sample_units(wl, 12, seed=layer)
    ref = oracle_ragged_units(inp, step, units)
    got, got_lse = gather_units(out, lse, wl, units)
    exp = np.stack([ref[u][0] for u in units])
    exp_lse = np.stack([ref[u][1] for u in units])
    assert_parity(got, exp, wl.dtype, f"c3 paged L{layer}", got_lse, exp_lse)
    assert_paged_writes(K, V, pc, step.to("cpu"), {u: ref[u][2] for u in units}, inp.raw_window,
                        units=units)
    del K, V, pc
    out_c, lse_c, _, _ = run_gpu_ragged(inp, step)
    assert np.array_equal(out, out_c) and np.array_equal(lse, lse_c)
    del inp
    torch.cuda.empty_cache()
