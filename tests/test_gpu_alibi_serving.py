"""The ALiBi forms of the serving calls against the fp64 oracle
(oracle.decode_chunk_alibi): slimkv_decode_attn_ragged_alibi, _paged_alibi,
_chunk_alibi and _chunk_paged_alibi.  Nothing is rotated; every score gets
-slope * (q_pos_t - k_pos) with beacons on a position grid, live raw rows
ending just before the new tokens (or at the query when there are none),
and new token u at q_pos + u.  The stored rows are the new tokens exactly
as given (no rotation), and nothing else in the cache changes."""

import dataclasses

import numpy as np
import pytest
import torch

import latent_decode_attention_amd as lda
import oracle
import synth
from parity_util import (assert_parity, note, ragged_edge_cases, ragged_workload, sample_units,
                         storage_bits)

pytestmark = pytest.mark.gpu


def params(wl, ratio=16, slopes=None):
    first, stride = synth.beacon_grid(ratio)
    sl = synth.alibi_slopes(wl.num_q_heads) if slopes is None else np.asarray(slopes)
    return np.asarray(sl, dtype=np.float32), first, stride


def run_alibi_serving(inp, tok, slopes, first, stride, *, Q=None, append=True, pc=None,
                      num_splits=0, device="cuda"):
    """One ALiBi serving call on the GPU: ragged (Q None, tok a StepInputs)
    or chunk (tok a ChunkInputs), over capacity arrays or the pages pc.  The
    raw arrays (or pools) are cloned first.  Returns out, lse, K, V (host)."""
    wl = inp.workload
    g = inp.to(device)
    t = tok.to(device)
    ncap, wcap = inp.num_beacons, inp.raw_window
    prob = lda.problem_from_tensors(g.q, g.U_K, g.C_K, g.K_raw, U_V=g.U_V,
                                    rope_theta=wl.rope_theta, num_kv_heads=wl.num_kv_heads,
                                    scale=wl.scale, num_splits=num_splits)
    sl = torch.as_tensor(slopes, device=device)
    al = lda.make_alibi(sl, first, stride)
    B, Hq, d = g.q.shape
    if pc is not None:
        bt, rt = pc.beacon_table.to(device), pc.raw_table.to(device)
        CK, CV = pc.C_K.to(device), pc.C_V.to(device)
        K, V = pc.K_raw.to(device).clone(), pc.V_raw.to(device).clone()
        pages = lda.make_pages(page_rows=pc.page_rows, beacon_table=bt if ncap else None,
                               raw_table=rt if wcap else None, beacon_pages=pc.beacon_pages,
                               raw_pages=pc.raw_pages)
    else:
        CK, CV = g.C_K, g.C_V
        K, V = g.K_raw.clone(), g.V_raw.clone()
    kn = t.k_new if append else None
    vn = t.v_new if append else None
    args = (g.U_K, g.U_V, CK if ncap else None, CV if ncap else None, K if wcap else None,
            V if wcap else None, t.num_beacons, t.raw_len, kn, vn)
    if Q is None:
        out, lse = lda.alloc_outputs(prob, device)
        ws = lda.alloc_workspace(prob, lda.SLIMKV_OP_LATENT_RAGGED, device)
        if pc is None:
            lda.slimkv_decode_attn_ragged_alibi(prob, al, g.q, g.q_pos, *args, out, lse, ws)
        else:
            lda.slimkv_decode_attn_paged_alibi(prob, pages, al, g.q, g.q_pos, *args, out, lse, ws)
    else:
        out = torch.empty((B, Q, Hq, d), dtype=torch.float32, device=device)
        lse = torch.empty((B, Q, Hq), dtype=torch.float32, device=device)
        ws = torch.zeros(lda.slimkv_chunk_workspace_bytes(prob, Q), dtype=torch.uint8, device=device)
        if pc is None:
            lda.slimkv_decode_attn_chunk_alibi(prob, al, Q, t.q, g.q_pos, *args, out, lse, ws)
        else:
            lda.slimkv_decode_attn_chunk_paged_alibi(prob, pages, al, Q, t.q, g.q_pos, *args, out,
                                                     lse, ws)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), lse.double().cpu().numpy(), K.cpu(), V.cpu()


def oracle_alibi_serving(inp, tok, slopes, first, stride, *, Q=None, append=True, units=None):
    wl = inp.workload
    st = synth.to_numpy_storage
    nb, w = inp.num_beacons, inp.raw_window
    bpos = (first + stride * np.arange(nb)).astype(np.int32)
    q = st(inp.q) if Q is None else st(tok.q)
    return oracle.decode_chunk_alibi(
        q, st(inp.q_pos), st(inp.U_K), st(inp.U_V), st(inp.C_K) if nb else None,
        st(inp.C_V) if nb else None, st(inp.K_raw) if w else None, st(inp.V_raw) if w else None,
        beacon_pos=bpos, slopes=slopes.astype(np.float64), num_kv_heads=wl.num_kv_heads,
        scale=wl.scale, num_beacons=st(tok.num_beacons), raw_len=st(tok.raw_len),
        k_new=st(tok.k_new) if append else None, v_new=st(tok.v_new) if append else None,
        units=units)


def assert_stored_as_given(K_after, V_after, K_before, V_before, tok, Q):
    """New token u of sequence b is row raw_len[b] + u of every KV head, bit
    for bit as given (while the window has room); nothing else changed."""
    Ka, Va = storage_bits(K_after), storage_bits(V_after)
    Kb, Vb = storage_bits(K_before), storage_bits(V_before)
    kn, vn = storage_bits(tok.k_new), storage_bits(tok.v_new)
    if Q is None:
        kn, vn = kn[:, None], vn[:, None]
    B, Hkv, wcap, d = Ka.shape
    mask = np.zeros((B, Hkv, wcap), dtype=bool)
    raw_len = tok.raw_len.cpu().numpy()
    for b in range(B):
        w = int(np.clip(raw_len[b], 0, wcap))
        for u in range(kn.shape[1]):
            if w + u < wcap:
                mask[b, :, w + u] = True
                assert np.array_equal(Ka[b, :, w + u], kn[b, u]), f"stored key ({b}, {u})"
                assert np.array_equal(Va[b, :, w + u], vn[b, u]), f"stored value ({b}, {u})"
    assert np.array_equal(Ka[~mask], Kb[~mask]) and np.array_equal(Va[~mask], Vb[~mask]), \
        "rows other than the new tokens' were written"


def check(wl, *, Q=None, append=True, page_rows=0, ratio=16, slopes=None, fixed=None,
          rank_v=None, num_splits=0, what=""):
    inp = synth.make_layer(wl, rank_v=rank_v)
    if Q is None:
        tok = synth.make_step(wl, inp, fixed=fixed if fixed is not None
                              else ragged_edge_cases(inp.num_beacons, inp.raw_window))
    else:
        tok = synth.make_chunk(wl, inp, Q, fixed=fixed)
    sl, first, stride = params(wl, ratio, slopes)
    pc = synth.make_paged(inp, tok, page_rows=page_rows) if page_rows else None
    note(f"alibi serving {what}: B={wl.batch} Hkv={wl.num_kv_heads} G={wl.group} "
         f"nb={inp.num_beacons} w={inp.raw_window} r=({inp.rank_k}, {inp.rank_v}) {wl.dtype} "
         f"Q={Q} append={append} pages={page_rows} splits={num_splits}")
    out, lse, K, V = run_alibi_serving(inp, tok, sl, first, stride, Q=Q, append=append, pc=pc,
                                       num_splits=num_splits)
    ref, ref_lse, _ = oracle_alibi_serving(inp, tok, sl, first, stride, Q=Q, append=append)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse)), f"{what}: rows with nothing to attend"
    assert_parity(out, ref, wl.dtype, what, lse[fin], ref_lse[fin])
    if append and pc is None:
        assert_stored_as_given(K, V, inp.K_raw, inp.V_raw, tok, Q)
    if append and pc is not None:
        # the pools as the contiguous call would have left them, paged again
        out_c, lse_c, Kc, Vc = run_alibi_serving(inp, tok, sl, first, stride, Q=Q, append=True,
                                                 num_splits=num_splits)
        assert np.array_equal(out, out_c) and np.array_equal(lse, lse_c), \
            f"{what}: paged call differs from the contiguous one"
    return out, lse


def small(dtype="bf16", B=6, Hkv=2, G=4, nb=700, w=300, r=64, index=190):
    return ragged_workload(dtype=dtype, B=B, Hkv=Hkv, G=G, nb=nb, w=w, r=r, index=index)


def test_ragged_bf16_edge_cases(gpu_device):
    check(small(), what="ragged bf16 G4")


def test_ragged_without_new_token(gpu_device):
    check(small(index=191), append=False, what="ragged no token")


@pytest.mark.parametrize("G,r,rv", [(1, 32, None), (5, 48, 96), (8, 128, None)])
def test_ragged_groups(G, r, rv, gpu_device):
    check(small(B=4, G=G, nb=500, w=130, r=r, index=192 + G), rank_v=rv, what=f"ragged G{G}")


def test_ragged_fp32(gpu_device):
    check(small(dtype="fp32", B=4, G=4, nb=300, w=80, r=32, index=200), what="ragged fp32")


def test_ragged_near_beacons(gpu_device):
    """Beacons right behind the window and gentle slopes: both segments and
    the token weigh in."""
    check(small(B=4, nb=200, w=64, index=201), ratio=1, slopes=np.full(8, 0.003),
          what="ragged near beacons")


@pytest.mark.parametrize("splits", [1, 7, 333])
def test_ragged_grids(splits, gpu_device):
    check(small(B=5, nb=900, w=200, index=202), num_splits=splits, what=f"ragged grid {splits}")


@pytest.mark.parametrize("page_rows", [64, 128])
def test_paged(page_rows, gpu_device):
    check(small(B=5, nb=800, w=300, index=203 + page_rows), page_rows=page_rows,
          what=f"paged {page_rows}")


@pytest.mark.parametrize("G,Q,r,rv", [(4, 4, 64, None), (8, 2, 32, None), (5, 3, 48, 96),
                                      (1, 16, 64, None)])
def test_chunk(G, Q, r, rv, gpu_device):
    check(small(B=4, G=G, nb=600, w=200, r=r, index=210 + G * Q), Q=Q, rank_v=rv,
          what=f"chunk G{G} Q{Q}")


@pytest.mark.parametrize("page_rows", [0, 64])
def test_chunk_fp32(page_rows, gpu_device):
    check(small(dtype="fp32", B=4, G=4, nb=300, w=90, r=32, index=230 + page_rows), Q=3,
          page_rows=page_rows, what=f"chunk fp32 pages {page_rows}")


def test_chunk_without_new_tokens(gpu_device):
    check(small(B=4, nb=500, w=150, index=220), Q=4, append=False, what="chunk no tokens")


def test_chunk_window_nearly_full(gpu_device):
    """Windows with room for only part of the chunk: the rest is attended
    but not stored."""
    wl = small(B=3, nb=400, w=100, index=221)
    check(wl, Q=4, fixed={0: (400, 98), 1: (10, 100), 2: (0, 0)}, what="chunk window full")


@pytest.mark.parametrize("page_rows", [64, 1024])
def test_chunk_paged(page_rows, gpu_device):
    check(small(B=4, nb=900, w=300, index=222 + page_rows), Q=4, page_rows=page_rows,
          what=f"chunk paged {page_rows}")


def test_zero_slopes_match_rotary_at_position_zero(gpu_device):
    """With zero slopes and every position at 0 the rotary ragged call rotates
    nothing either (query and new key turn by angle 0): the two calls agree."""
    wl = small(B=4, nb=300, w=100, index=230)
    inp = synth.make_layer(wl)
    inp.q_pos = torch.zeros_like(inp.q_pos)
    tok = synth.make_step(wl, inp)
    sl, first, stride = params(wl, slopes=np.zeros(wl.num_q_heads))
    note("alibi zero slopes vs rotary at position 0")
    out, lse, _, _ = run_alibi_serving(inp, tok, sl, 0, 0)
    g, t = inp.to("cuda"), tok.to("cuda")
    prob = lda.problem_from_tensors(g.q, g.U_K, g.C_K, g.K_raw, U_V=g.U_V, rope_theta=wl.rope_theta,
                                    num_kv_heads=wl.num_kv_heads, scale=wl.scale)
    o2, l2 = lda.alloc_outputs(prob, "cuda")
    ws = lda.alloc_workspace(prob, lda.SLIMKV_OP_LATENT_RAGGED, "cuda")
    lda.slimkv_decode_attn_ragged(prob, g.q, g.q_pos, g.U_K, g.U_V, g.C_K, g.C_V, g.K_raw.clone(),
                                  g.V_raw.clone(), t.num_beacons, t.raw_len, t.k_new, t.v_new, o2, l2,
                                  ws)
    torch.cuda.synchronize()
    assert_parity(out, o2.double().cpu().numpy(), "bf16", "zero slopes vs rotary",
                  lse, l2.double().cpu().numpy())


@pytest.mark.parametrize("layer", [1, 6])  # ranks 64, 128
def test_c3_layers_sampled(layer, gpu_device):
    """The c3 serving step as an ALiBi backbone runs it (75% of the rows
    live, a new token), on sampled units."""
    wl = synth.get_workload("c3")
    note(f"alibi serving c3 layer {layer} (generate on GPU)")
    inp = synth.make_layer(wl, layer, device="cuda")
    tok = synth.make_step(wl, inp, device="cuda", beacons=(0.5, 1.0), raw=(0.5, 1.0))
    sl, first, stride = params(wl)
    out, lse, _, _ = run_alibi_serving(inp, tok, sl, first, stride)
    units = sample_units(wl, 6, layer)
    G = wl.group
    got = np.stack([out[b, h * G:(h + 1) * G] for b, h in units])
    got_l = np.stack([lse[b, h * G:(h + 1) * G] for b, h in units])
    ref, ref_lse, _ = oracle_alibi_serving(inp, tok, sl, first, stride, units=units)
    exp = np.stack([ref[b, h * G:(h + 1) * G] for b, h in units])
    exp_l = np.stack([ref_lse[b, h * G:(h + 1) * G] for b, h in units])
    assert_parity(got, exp, "bf16", f"alibi serving c3 L{layer}", got_l, exp_l)
