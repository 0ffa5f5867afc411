"""The serving entry points under HIP graph capture: ragged, paged, chunk,
paged chunk and ALiBi calls captured together as one graph.  Every replay -- with eager
calls and synchronisation between replays -- reproduces the eager outputs
and cache rows bit for bit (the library records no memset, allocates
nothing, and leaves its workspace counters at zero after each call)."""

import numpy as np
import pytest
import torch

import latent_decode_attention_amd as lda
import synth
from parity_util import note
from parity_util import ragged_edge_cases as edge_cases
from parity_util import ragged_workload as custom

pytestmark = pytest.mark.gpu


def test_graph_replays_of_serving_calls(gpu_device):
    dev = "cuda"
    wl = custom(B=6, Hkv=2, G=4, nb=700, w=150, index=190)
    inp = synth.make_layer(wl).to(dev)
    step = synth.make_step(wl, inp, device=dev, fixed=edge_cases(700, 150))
    pc = synth.make_paged(inp, step, page_rows=64)
    ch = synth.make_chunk(wl, inp, 4, device=dev, fixed=edge_cases(700, 150))
    pc2 = synth.make_paged(inp, ch, page_rows=64)
    prob = lda.problem_from_tensors(inp.q, inp.U_K, inp.C_K, inp.K_raw, U_V=inp.U_V,
                                    rope_theta=wl.rope_theta, num_kv_heads=wl.num_kv_heads,
                                    scale=wl.scale)
    pages = lda.make_pages(page_rows=64, beacon_table=pc.beacon_table, raw_table=pc.raw_table,
                           beacon_pages=pc.beacon_pages, raw_pages=pc.raw_pages)
    K1, V1 = inp.K_raw.clone(), inp.V_raw.clone()        # written by the ragged call
    K2, V2 = pc.K_raw.clone(), pc.V_raw.clone()          # written by the paged call
    K3, V3 = inp.K_raw.clone(), inp.V_raw.clone()        # written by the chunk call
    K4, V4 = pc2.K_raw.clone(), pc2.V_raw.clone()        # written by the paged chunk call
    pages2 = lda.make_pages(page_rows=64, beacon_table=pc2.beacon_table, raw_table=pc2.raw_table,
                            beacon_pages=pc2.beacon_pages, raw_pages=pc2.raw_pages)
    ws = [lda.alloc_workspace(prob, lda.SLIMKV_OP_LATENT_RAGGED, dev) for _ in range(2)]
    ws.append(torch.zeros(lda.slimkv_chunk_workspace_bytes(prob, 4), dtype=torch.uint8, device=dev))
    ws.append(lda.alloc_workspace(prob, lda.SLIMKV_OP_LATENT, dev))
    ws.append(torch.zeros(lda.slimkv_chunk_workspace_bytes(prob, 4), dtype=torch.uint8, device=dev))
    outs = [lda.alloc_outputs(prob, dev) for _ in range(2)]
    B, Hq, d = inp.q.shape
    outs.append((torch.empty((B, 4, Hq, d), device=dev), torch.empty((B, 4, Hq), device=dev)))
    outs.append(lda.alloc_outputs(prob, dev))
    outs.append((torch.empty((B, 4, Hq, d), device=dev), torch.empty((B, 4, Hq), device=dev)))
    slopes = torch.as_tensor(synth.alibi_slopes(Hq).astype(np.float32), device=dev)
    note("graph capture of ragged, paged, chunk, paged chunk and ALiBi calls")

    def run():
        lda.slimkv_decode_attn_ragged(prob, inp.q, inp.q_pos, inp.U_K, inp.U_V, inp.C_K, inp.C_V,
                                      K1, V1, step.num_beacons, step.raw_len, step.k_new,
                                      step.v_new, *outs[0], ws[0])
        lda.slimkv_decode_attn_paged(prob, pages, inp.q, inp.q_pos, inp.U_K, inp.U_V, pc.C_K,
                                     pc.C_V, K2, V2, step.num_beacons, step.raw_len, step.k_new,
                                     step.v_new, *outs[1], ws[1])
        lda.slimkv_decode_attn_chunk(prob, 4, ch.q, inp.q_pos, inp.U_K, inp.U_V, inp.C_K, inp.C_V,
                                     K3, V3, ch.num_beacons, ch.raw_len, ch.k_new, ch.v_new,
                                     *outs[2], ws[2])
        lda.slimkv_decode_attn_alibi(prob, inp.q, inp.q_pos, inp.U_K, inp.U_V, inp.C_K, inp.C_V,
                                     inp.K_raw, inp.V_raw, slopes, 15, 16, *outs[3], ws[3])
        lda.slimkv_decode_attn_chunk_paged(prob, pages2, 4, ch.q, inp.q_pos, inp.U_K, inp.U_V,
                                           pc2.C_K, pc2.C_V, K4, V4, ch.num_beacons, ch.raw_len,
                                           ch.k_new, ch.v_new, *outs[4], ws[4])

    run()
    torch.cuda.synchronize()
    ref = [(o.clone(), l.clone()) for o, l in outs]
    caches = [K1.clone(), V1.clone(), K2.clone(), V2.clone(), K3.clone(), V3.clone(), K4.clone(),
              V4.clone()]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for _ in range(4):
        for o, l in outs:
            o.zero_()
            l.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for (o, l), (ro, rl) in zip(outs, ref):
            assert torch.equal(o, ro) and torch.equal(l, rl)
        for c, rc in zip((K1, V1, K2, V2, K3, V3, K4, V4), caches):  # (pools hold NaN fillers)
            assert torch.equal(c.view(torch.int16), rc.view(torch.int16))
        run()  # eager work between replays
        torch.cuda.synchronize()
