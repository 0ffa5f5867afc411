"""slimkv_decode_attn_noalloc (the entry point that allocates nothing; its
workspace is a scratch array inside the library) against
slimkv_decode_attn with a caller's workspace, through the C ABI: two calls
in a row, the second on a smaller input, each equal to the workspace call
bit for bit and within the bf16 / fp32 bars of the fp64 oracle; a problem
too large for the scratch is refused before any launch."""

import dataclasses

import pytest
import torch

import latent_decode_attention_amd as lda
import synth
from parity_util import assert_parity, note, oracle_layer

pytestmark = pytest.mark.gpu


def custom(dtype="bf16", B=2, Hkv=2, G=4, nb=100, w=37, r=64, index=95):
    return dataclasses.replace(
        synth.get_workload("c2"), name="custom", index=index, batch=B, num_q_heads=Hkv * G,
        num_kv_heads=Hkv, num_beacons=nb, raw_window=w, ranks=(r,), dtype=dtype, sigma=1.0,
        rope_theta=5e5, context=4096)


def both_calls(inp, num_splits=0):
    """(noalloc out, lse), (workspace out, lse) on the GPU for one layer."""
    wl = inp.workload
    g = inp.to("cuda")
    prob = lda.problem_from_tensors(g.q, g.U_K, g.C_K, g.K_raw, U_V=g.U_V,
                                    rope_theta=wl.rope_theta, num_kv_heads=wl.num_kv_heads,
                                    scale=wl.scale, num_splits=num_splits)
    out_n, lse_n = lda.alloc_outputs(prob, "cuda")
    out_n.fill_(float("nan"))
    lda.slimkv_decode_attn_noalloc(prob, g.q, g.q_pos, g.U_K, g.U_V, g.C_K, g.C_V, g.K_raw,
                                   g.V_raw, out_n, lse_n)
    torch.cuda.synchronize()
    out_w, lse_w = lda.alloc_outputs(prob, "cuda")
    ws = lda.alloc_workspace(prob, lda.SLIMKV_OP_LATENT, "cuda")
    lda.slimkv_decode_attn(prob, g.q, g.q_pos, g.U_K, g.U_V, g.C_K, g.C_V, g.K_raw, g.V_raw,
                           out_w, lse_w, ws)
    torch.cuda.synchronize()
    return (out_n, lse_n), (out_w, lse_w)


def check(inp, what, num_splits=0):
    wl = inp.workload
    note(f"noalloc {what}: B={wl.batch} Hkv={wl.num_kv_heads} G={wl.group} nb={inp.num_beacons} "
         f"w={inp.raw_window} r={inp.rank_k} {wl.dtype} splits={num_splits}")
    (out_n, lse_n), (out_w, lse_w) = both_calls(inp, num_splits)
    assert torch.equal(out_n, out_w), f"{what}: out differs from the workspace call"
    assert torch.equal(lse_n, lse_w), f"{what}: lse differs from the workspace call"
    ref, ref_lse = oracle_layer(inp)
    assert_parity(out_n.double().cpu().numpy(), ref, wl.dtype, what,
                  lse_n.double().cpu().numpy(), ref_lse)


def test_two_calls_second_smaller(gpu_device):
    check(synth.make_layer(custom(B=8, Hkv=4, G=4, nb=3000, w=700, r=64)), "first (larger)")
    check(synth.make_layer(custom(B=2, Hkv=2, G=5, nb=500, w=130, r=48, index=96)),
          "second (smaller)")


def test_forced_splits_and_fp32(gpu_device):
    check(synth.make_layer(custom(B=3, Hkv=2, G=8, nb=2000, w=65, r=32, index=97)), "64 splits",
          num_splits=64)
    check(synth.make_layer(custom(dtype="fp32", B=2, Hkv=1, G=4, nb=512, w=128, r=32, index=98)),
          "fp32")


def test_c3_layer_sampled(gpu_device):
    """A 128K layer of the benchmark's step (rank 128, the widest), bitwise
    against the workspace call (which the parity tests hold to the oracle)."""
    wl = synth.get_workload("c3")
    layer = wl.ranks.index(128)
    inp = synth.make_layer(wl, layer, device="cuda")
    note(f"noalloc c3 layer {layer}")
    (out_n, lse_n), (out_w, lse_w) = both_calls(inp)
    assert torch.equal(out_n, out_w) and torch.equal(lse_n, lse_w)


def test_too_large_is_refused(gpu_device):
    """A problem whose partials exceed the scratch returns
    SLIMKV_ERR_WORKSPACE and leaves out untouched."""
    wl = custom(B=1024, Hkv=8, G=8, nb=64, w=0, r=16, index=99)
    prob = lda.make_problem(batch=wl.batch, num_q_heads=wl.num_q_heads,
                            num_kv_heads=wl.num_kv_heads, num_beacons=wl.num_beacons, rank_k=16,
                            rank_v=16, raw_window=0, scale=wl.scale, rope_theta=wl.rope_theta,
                            dtype="bf16", num_splits=2)
    q = torch.zeros(wl.batch, wl.num_q_heads, 128, dtype=torch.bfloat16, device="cuda")
    q_pos = torch.zeros(wl.batch, dtype=torch.int32, device="cuda")
    U = torch.zeros(wl.num_kv_heads, 128, 16, dtype=torch.bfloat16, device="cuda")
    C = torch.zeros(wl.batch, wl.num_kv_heads, 64, 16, dtype=torch.bfloat16, device="cuda")
    out, lse = lda.alloc_outputs(prob, "cuda")
    out.fill_(7.0)
    with pytest.raises(lda.SlimKVError) as e:
        lda.slimkv_decode_attn_noalloc(prob, q, q_pos, U, U.clone(), C, C.clone(), None, None, out,
                                       lse)
    assert e.value.status == 4 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
