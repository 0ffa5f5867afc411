"""HIP library vs the fp64 oracle, element by element, on seeded inputs.

Small configurations are compared over the whole output; the 128K
workloads, run in the launch configuration the benchmark times, are
compared on sampled (b, kv head) units the oracle computes one by one.
"""

import dataclasses

import numpy as np
import pytest
import torch

import latent_decode_attention_amd as lda
import synth
from parity_util import (RECON_LSE_TOL, assert_parity, beacon_positions, gather_units, note,
                         oracle_full_kv_units, oracle_layer, oracle_units, run_gpu, sample_units)

pytestmark = pytest.mark.gpu

LAT, REC, FULL = lda.SLIMKV_OP_LATENT, lda.SLIMKV_OP_RECONSTRUCT, lda.SLIMKV_OP_FULL_KV
# The workspace opens with a 256-byte header (word 0: the status word of
# SLIMKV_FLAG_CHECK_WORKSPACE), then one 64-byte line of counters per
# (b, kv head) unit: 16 uint32, of which the first two are used.
WS_HEADER = 256
COUNTER_STRIDE = 16


def custom(dtype="bf16", B=2, Hkv=2, G=4, nb=100, w=37, r=64, sigma=1.0, theta=5e5,
           context=4096, index=90):
    return dataclasses.replace(
        synth.get_workload("c2"), name="custom", index=index, batch=B, num_q_heads=Hkv * G,
        num_kv_heads=Hkv, num_beacons=nb, raw_window=w, ranks=(r,), dtype=dtype, sigma=sigma,
        rope_theta=theta, context=context)


def check_full_layer(inp, op=LAT, what="", **kw):
    note(f"{what} op={op} B={inp.workload.batch} Hkv={inp.workload.num_kv_heads} "
         f"G={inp.workload.group} nb={inp.num_beacons} w={inp.raw_window} "
         f"rk={inp.rank_k} rv={inp.rank_v} {inp.workload.dtype}")
    out, lse = run_gpu(inp, op, **kw)
    ref, ref_lse = oracle_layer(inp)
    lse_tol = RECON_LSE_TOL[inp.workload.dtype] if op == REC else None
    assert_parity(out, ref, inp.workload.dtype, what, lse, ref_lse, lse_tol=lse_tol)
    return out, lse


def test_c1_fp32_full(gpu_device):
    inp = synth.make_layer(synth.get_workload("c1"))
    check_full_layer(inp, what="c1")


def test_c2_bf16_full(gpu_device):
    inp = synth.make_layer(synth.get_workload("c2"))
    check_full_layer(inp, what="c2")


RAGGED = [
    # dtype, B, Hkv, G, nb, w, rk, rv
    ("bf16", 1, 1, 1, 1, 0, 16, 16),
    ("bf16", 1, 1, 4, 0, 1, 32, 32),
    ("bf16", 2, 3, 4, 17, 5, 32, 32),
    ("bf16", 1, 2, 5, 333, 129, 48, 48),
    ("bf16", 2, 1, 8, 64, 64, 64, 64),
    ("bf16", 1, 2, 3, 250, 0, 80, 80),
    ("bf16", 2, 2, 2, 97, 200, 96, 96),
    ("bf16", 1, 1, 7, 1000, 31, 112, 112),
    ("bf16", 1, 2, 6, 515, 77, 128, 128),
    ("bf16", 2, 2, 4, 300, 50, 32, 128),
    ("bf16", 1, 2, 5, 300, 50, 128, 16),
    ("bf16", 1, 1, 4, 4097, 1, 48, 96),
    ("fp32", 1, 1, 4, 33, 17, 32, 32),
    ("fp32", 2, 2, 5, 200, 3, 48, 128),
    ("fp32", 1, 2, 8, 0, 100, 64, 64),
    ("fp32", 1, 1, 1, 129, 0, 128, 16),
]


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: "-".join(map(str, c)))
def test_ragged_shapes(case, gpu_device):
    dtype, B, Hkv, G, nb, w, rk, rv = case
    wl = custom(dtype=dtype, B=B, Hkv=Hkv, G=G, nb=nb, w=w, r=rk, index=91)
    inp = synth.make_layer(wl, rank_v=rv)
    check_full_layer(inp, what=f"ragged {case}")


@pytest.mark.parametrize("case", RAGGED[::3], ids=lambda c: "-".join(map(str, c)))
def test_ragged_reconstruct(case, gpu_device):
    dtype, B, Hkv, G, nb, w, rk, rv = case
    wl = custom(dtype=dtype, B=B, Hkv=Hkv, G=G, nb=nb, w=w, r=rk, index=92)
    inp = synth.make_layer(wl, rank_v=rv)
    check_full_layer(inp, REC, what=f"reconstruct {case}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_full_kv_small(dtype, gpu_device):
    wl = custom(dtype=dtype, B=2, Hkv=2, G=4, nb=0, w=0, context=2048, index=93)
    k, v = synth.make_full_kv(wl)
    inp = synth.make_layer(wl, num_beacons=0, raw_window=wl.context)
    assert torch.equal(inp.K_raw, k)
    note(f"full_kv small {dtype}")
    out, lse = run_gpu(inp, FULL, full_k=k, full_v=v)
    ref, ref_lse = oracle_layer(inp)
    assert_parity(out, ref, dtype, f"full-kv {dtype}", lse, ref_lse)


def test_split_counts_agree(gpu_device):
    wl = custom(B=2, Hkv=2, G=4, nb=1500, w=300, r=64, index=94)
    inp = synth.make_layer(wl)
    ref, ref_lse = oracle_layer(inp)
    outs = []
    for splits in (1, 2, 7, 4096):
        note(f"splits={splits}")
        out, lse = run_gpu(inp, LAT, num_splits=splits)
        assert_parity(out, ref, "bf16", f"splits={splits}", lse, ref_lse)
        outs.append(out)
    for o in outs[1:]:
        rel = np.linalg.norm(o - outs[0]) / np.linalg.norm(outs[0])
        assert rel < 1e-5, rel


def test_large_scores_and_needles(gpu_device):
    """Query scaled x30 (scores in the hundreds), plus a beacon and a raw key
    placed in the last chunk that line up with the query: the online
    softmax must rescale without overflow and find them."""
    wl = custom(B=1, Hkv=2, G=4, nb=2000, w=500, r=64, index=95)
    inp = synth.make_layer(wl)
    inp.q = (inp.q.float() * 30).to(inp.q.dtype)
    # needle beacon: latent key = U_K^T of the rotated query of head 0 (up to scale);
    # a large multiple of the first basis direction is enough to dominate
    inp.C_K[0, 0, -1] = (inp.C_K[0, 0, -1].float() * 0 + 8.0).to(inp.C_K.dtype)
    inp.K_raw[0, 1, -1] = (inp.K_raw[0, 1, -1].float() * 6).to(inp.K_raw.dtype)
    check_full_layer(inp, what="stress x30 + needles")
    check_full_layer(inp, what="stress x30 + needles, 1 split", num_splits=1)


def test_constant_values_give_exact_ones(gpu_device):
    """All value rows equal to ones => every output is 1 (weights sum to 1)."""
    wl = custom(B=2, Hkv=2, G=4, nb=300, w=70, r=32, index=96)
    inp = synth.make_layer(wl)
    d, r = 128, 32
    rng = np.random.default_rng(0)
    basis = np.concatenate([np.ones((d, 1)) / np.sqrt(d), rng.standard_normal((d, r - 1))], 1)
    uv, rm = np.linalg.qr(basis)
    uv = uv * np.sign(np.diag(rm))
    # bf16 basis: first column exactly 2^-k-representable scaled ones
    col0 = torch.full((d,), 1.0 / 16.0)  # 1/sqrt(256) keeps bf16 exact; C_V[...,0] = 16
    u = torch.from_numpy(uv).float()
    u[:, 0] = col0
    inp.U_V = torch.stack([u, u]).to(inp.U_V.dtype)
    cv = torch.zeros_like(inp.C_V)
    cv[..., 0] = 16.0
    inp.C_V = cv
    inp.V_raw = torch.ones_like(inp.V_raw)
    note("constant values")
    out, _ = run_gpu(inp, LAT)
    # fp32 sums plus the two-term bf16 split of the latent sum before the U_V
    # lift (2^-17 relative) bound the error near 1e-5; a normalisation mistake
    # (separate softmaxes, a dropped branch) is off by O(1).
    assert np.abs(out - 1.0).max() < 1e-5, np.abs(out - 1.0).max()


def test_repeat_calls_identical_and_lse_optional(gpu_device):
    """By default repeated calls are bitwise equal; with tiles taken from a
    shared counter they agree to rounding."""
    inp = synth.make_layer(custom(B=2, Hkv=2, G=5, nb=700, w=90, r=48, index=97))
    note("determinism")
    a, la = run_gpu(inp, LAT)
    b, lb = run_gpu(inp, LAT)
    c, lc = run_gpu(inp, LAT, with_lse=False)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    assert np.array_equal(a, c) and lc is None
    for _ in range(3):
        d, ld = run_gpu(inp, LAT, flags=lda.SLIMKV_FLAG_DYNAMIC_TILES)
        assert np.abs(d - a).max() <= 1e-5 * np.abs(a).max()
        assert np.abs(ld - la).max() <= 1e-5


def _sampled(wl, layer, op=LAT, n_units=6, seed=0):
    note(f"{wl.name} layer {layer} op={op} (generate on GPU)")
    inp = synth.make_layer(wl, layer, device="cuda")
    units = sample_units(wl, n_units, seed + layer)
    out, lse = run_gpu(inp, op)
    ref = oracle_units(inp, units)
    got, got_lse = gather_units(out, lse, wl, units)
    exp = np.stack([ref[u][0] for u in units])
    exp_lse = np.stack([ref[u][1] for u in units])
    assert_parity(got, exp, wl.dtype, f"{wl.name} L{layer} op{op} {len(units)} units", got_lse,
                  exp_lse, lse_tol=RECON_LSE_TOL[wl.dtype] if op == REC else None)
    del inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layer", [0, 6, 13, 3])  # ranks 48, 128, 96, 32
def test_c3_sampled(layer, gpu_device):
    _sampled(synth.get_workload("c3"), layer)


@pytest.mark.parametrize("layer", [0, 1, 9])  # ranks 32, 128, 48 with G = 5
def test_c4_sampled(layer, gpu_device):
    _sampled(synth.get_workload("c4"), layer)


@pytest.mark.parametrize("key", ["c5_4x", "c5_32x"])
def test_c5_latent_sampled(key, gpu_device):
    _sampled(synth.get_workload(key), 0, n_units=4)


def test_c5_reconstruct_sampled(gpu_device):
    _sampled(synth.get_workload("c5_16x"), 0, op=REC, n_units=4)


def test_c5_full_kv_sampled(gpu_device):
    wl = synth.get_workload("c5_full")
    note("c5 full-KV 131072 tokens (generate on GPU)")
    k, v = synth.make_full_kv(wl, 0, device="cuda")
    inp = synth.make_layer(wl, 0, device="cuda", num_beacons=0, raw_window=128)
    out, lse = run_gpu(inp, FULL, full_k=k, full_v=v)
    units = sample_units(wl, 3, 5)
    ref = oracle_full_kv_units(wl, inp.q, inp.q_pos, k, v, units)
    got, got_lse = gather_units(out, lse, wl, units)
    assert_parity(got, np.stack([ref[u][0] for u in units]), "bf16", "c5 full-KV", got_lse,
                  np.stack([ref[u][1] for u in units]))


def test_workspace_reused_across_plans(gpu_device):
    """One workspace, many calls with different split plans and shapes: the
    per-unit counters the last chunk resets must leave it ready each time."""
    wl = custom(B=2, Hkv=2, G=4, nb=900, w=120, r=64, index=98)
    inp = synth.make_layer(wl)
    g = inp.to("cuda")
    ref, ref_lse = oracle_layer(inp)
    ws = None
    for splits in (7, 1, 3, 0, 64, 2):
        prob = lda.problem_from_tensors(g.q, g.U_K, g.C_K, g.K_raw, U_V=g.U_V,
                                        rope_theta=wl.rope_theta, num_kv_heads=wl.num_kv_heads,
                                        scale=wl.scale, num_splits=splits)
        need = lda.slimkv_workspace_bytes(prob, LAT)
        if ws is None:
            ws = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")
        assert need <= ws.numel()
        out, lse = lda.alloc_outputs(prob, "cuda")
        note(f"workspace reuse splits={splits}")
        lda.slimkv_decode_attn(prob, g.q, g.q_pos, g.U_K, g.U_V, g.C_K, g.C_V, g.K_raw, g.V_raw,
                               out, lse, ws)
        torch.cuda.synchronize()
        assert_parity(out.double().cpu().numpy(), ref, "bf16", f"reuse splits={splits}",
                      lse.double().cpu().numpy(), ref_lse)
    # every unit's counter line (16 uint32 per unit: workgroups done, tiles
    # handed out, the rest unused) and every partial slot's flag (one uint32
    # per slot, 64 slots per unit, from the next 256-byte boundary) are back
    # at zero
    units = wl.batch * wl.num_kv_heads
    c0 = WS_HEADER
    counters = ws[c0:c0 + COUNTER_STRIDE * 4 * units].view(torch.int32).view(units, COUNTER_STRIDE)
    assert int(counters.abs().sum()) == 0, counters[counters.abs().sum(dim=1) != 0]
    f0 = (c0 + COUNTER_STRIDE * 4 * units + 255) // 256 * 256
    flags = ws[f0:f0 + 64 * 4 * units].view(torch.int32)
    assert int(flags.abs().sum()) == 0, torch.nonzero(flags)
    assert lda.slimkv_workspace_status(ws) == 0


def test_workspace_check_flag(gpu_device):
    """SLIMKV_FLAG_CHECK_WORKSPACE: a workspace whose counters and flags
    hold garbage (as one left by an interrupted call would) still gives the
    right result, and the status word reports it; a clean workspace keeps
    the status at zero."""
    wl = custom(B=2, Hkv=2, G=4, nb=700, w=90, r=64, index=97)
    inp = synth.make_layer(wl)
    g = inp.to("cuda")
    ref, ref_lse = oracle_layer(inp)
    prob = lda.problem_from_tensors(g.q, g.U_K, g.C_K, g.K_raw, U_V=g.U_V,
                                    rope_theta=wl.rope_theta, num_kv_heads=wl.num_kv_heads,
                                    scale=wl.scale, num_splits=5,
                                    flags=lda.SLIMKV_FLAG_CHECK_WORKSPACE)
    ws = lda.alloc_workspace(prob, LAT, "cuda")
    units = wl.batch * wl.num_kv_heads
    out, lse = lda.alloc_outputs(prob, "cuda")
    note("workspace check: clean workspace")
    lda.slimkv_decode_attn(prob, g.q, g.q_pos, g.U_K, g.U_V, g.C_K, g.C_V, g.K_raw, g.V_raw,
                           out, lse, ws)
    torch.cuda.synchronize()
    assert lda.slimkv_workspace_status(ws) == 0
    assert_parity(out.double().cpu().numpy(), ref, "bf16", "check flag clean",
                  lse.double().cpu().numpy(), ref_lse)
    # plant garbage in every unit's done counter and in one partial flag
    c0 = WS_HEADER
    ws[c0:c0 + COUNTER_STRIDE * 4 * units].view(torch.int32).view(units, COUNTER_STRIDE)[:, 0] = 3
    f0 = (c0 + COUNTER_STRIDE * 4 * units + 255) // 256 * 256
    ws[f0:f0 + 4].view(torch.int32)[0] = 1
    out.fill_(float("nan"))
    note("workspace check: planted counters")
    lda.slimkv_decode_attn(prob, g.q, g.q_pos, g.U_K, g.U_V, g.C_K, g.C_V, g.K_raw, g.V_raw,
                           out, lse, ws)
    torch.cuda.synchronize()
    assert lda.slimkv_workspace_status(ws) == 1
    assert_parity(out.double().cpu().numpy(), ref, "bf16", "check flag planted",
                  lse.double().cpu().numpy(), ref_lse)
    counters = ws[c0:c0 + COUNTER_STRIDE * 4 * units].view(torch.int32)
    assert int(counters.abs().sum()) == 0


def test_many_chunks_repeatable(gpu_device):
    """Forty back-to-back calls with many workgroups per unit on one
    workspace, alternating the two schedules: every merge saw every
    workgroup's partial, and the counters were left at zero each time."""
    wl = custom(B=4, Hkv=4, G=4, nb=6000, w=900, r=64, index=99)
    inp = synth.make_layer(wl)
    g = inp.to("cuda")
    probs = [lda.problem_from_tensors(g.q, g.U_K, g.C_K, g.K_raw, U_V=g.U_V,
                                      rope_theta=wl.rope_theta, num_kv_heads=wl.num_kv_heads,
                                      scale=wl.scale, num_splits=48, flags=f)
             for f in (0, lda.SLIMKV_FLAG_DYNAMIC_TILES)]
    ws = lda.alloc_workspace(probs[0], LAT, "cuda")
    outs = []
    note("many chunks x40, both schedules, one workspace")
    for i in range(40):
        out, lse = lda.alloc_outputs(probs[0], "cuda")
        lda.slimkv_decode_attn(probs[i % 2], g.q, g.q_pos, g.U_K, g.U_V, g.C_K, g.C_V, g.K_raw,
                               g.V_raw, out, lse, ws)
        outs.append((out, lse))
    torch.cuda.synchronize()
    ref, ref_lse = oracle_layer(inp)
    assert_parity(outs[0][0].double().cpu().numpy(), ref, "bf16", "many chunks",
                  outs[0][1].double().cpu().numpy(), ref_lse)
    scale = outs[0][0].abs().max().item()
    for i, (o, l) in enumerate(outs[1:], start=1):
        if i % 2 == 0:  # fixed schedule: bitwise equal
            assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
        else:           # counter schedule: equal up to summation order
            assert (o - outs[0][0]).abs().max().item() <= 1e-5 * scale
            assert (l - outs[0][1]).abs().max().item() <= 1e-5


def test_graph_replays_match_eager(gpu_device):
    """Several layer calls captured as one HIP graph: every replay, with eager
    calls and synchronisation between replays, reproduces the eager outputs
    bit for bit (the library records no memset and allocates nothing)."""
    wl = dataclasses.replace(custom(B=3, Hkv=2, G=4, nb=1500, w=300, index=96), layers=3,
                             ranks=(48, 64, 32))
    layers = [synth.make_layer(wl, layer=l).to("cuda") for l in range(3)]
    probs = [lda.problem_from_tensors(x.q, x.U_K, x.C_K, x.K_raw, U_V=x.U_V, rope_theta=wl.rope_theta,
                                      num_kv_heads=wl.num_kv_heads, scale=wl.scale) for x in layers]
    ws = lda.alloc_workspace(probs[0], LAT, "cuda")
    outs = [lda.alloc_outputs(p, "cuda") for p in probs]
    note("graph capture and replay")

    def step():
        for p, x, (o, l) in zip(probs, layers, outs):
            lda.slimkv_decode_attn(p, x.q, x.q_pos, x.U_K, x.U_V, x.C_K, x.C_V, x.K_raw, x.V_raw,
                                   o, l, ws)

    step()
    torch.cuda.synchronize()
    ref = [(o.clone(), l.clone()) for o, l in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(4):
        for o, l in outs:
            o.zero_()
            l.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for (o, l), (ro, rl) in zip(outs, ref):
            assert torch.equal(o, ro) and torch.equal(l, rl)
        step()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("dtype,G,nb,w,rk,rv", [("bf16", 4, 300, 50, 64, 64),
                                               ("bf16", 5, 777, 17, 48, 96),
                                               ("fp32", 4, 200, 33, 32, 32)])
def test_reconstruct_rope_small(dtype, G, nb, w, rk, rv, gpu_device):
    """The reconstruction variant that rotates rebuilt beacon keys at their
    positions (16x spacing), whole output against the oracle."""
    inp = synth.make_layer(custom(dtype=dtype, B=2, Hkv=2, G=G, nb=nb, w=w, r=rk, index=91,
                                  context=nb * 16), rank_v=rv)
    pos = beacon_positions(nb, nb * 16)
    note(f"reconstruct-rope {dtype} G={G} nb={nb} w={w} r=({rk},{rv})")
    out, lse = run_gpu(inp, REC, beacon_pos=pos)
    ref, ref_lse = oracle_layer(inp, beacon_pos=pos)
    assert_parity(out, ref, dtype, "reconstruct-rope", lse, ref_lse,
                  lse_tol=RECON_LSE_TOL[dtype])
    lat, _ = oracle_layer(inp)
    assert np.max(np.abs(ref - lat)) > 1e-3  # the rotation matters: not the latent result


def test_c5_reconstruct_rope_sampled(gpu_device):
    wl = synth.get_workload("c5_16x")
    note("c5_16x reconstruct-rope sampled")
    inp = synth.make_layer(wl, 0, device=gpu_device)
    pos = beacon_positions(wl.num_beacons, wl.context)
    out, lse = run_gpu(inp, REC, beacon_pos=pos)
    units = sample_units(wl, 10, seed=5)
    ref = oracle_units(inp, units, beacon_pos=pos)
    got, got_lse = gather_units(out, lse, wl, units)
    assert_parity(got, np.stack([ref[u][0] for u in units]), wl.dtype, "c5 reconstruct-rope",
                  got_lse, np.stack([ref[u][1] for u in units]), lse_tol=RECON_LSE_TOL[wl.dtype])
    del inp
    torch.cuda.empty_cache()

