#!/usr/bin/env python3
"""Decode-attention benchmark for libslimkv on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3]
                    [--no-cpu-baseline] [--no-compare] [--eager]

A step is one decode token's attention over every layer of the workload:
for the default workload (Llama-3.1-8B shape, 128K context, 16x token
compression, batch 16) that is 32 calls of slimkv_decode_attn, one per
layer, each with its own latent rank.  All inputs are generated on the GPU
before timing and stay resident in HBM.  The step's calls are captured once
as a HIP graph and replayed (checked bit for bit against the eager step;
--eager launches them directly).  The timed region is bracketed by device
synchronisation and measured with events on the stream the library
launches on.  Prints ONE JSON line.

Reported beside the headline tokens/s:
  * roofline of the sweep kernel (algorithmic cache bytes per launch over
    its average launch time, against 8 TB/s);
  * the comparison at 128K on one layer: latent path at 16x vs the
    reconstruct-then-attend paths on the same beacons (without and with the
    rotation of rebuilt beacon keys) and vs uncompressed full-KV attention
    over all 131072 tokens; the ragged serving step, over capacity-sized
    arrays and over a paged cache, and with 4 query tokens per sequence;
    the same step as an ALiBi backbone runs it; the 48-layer Qwen step;
  * the fp64 CPU oracle timed on a bounded sample on this host's cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import pathlib
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--eager", action="store_true",
                    help="launch each step's calls directly instead of replaying the step as one "
                         "captured HIP graph")
    ap.add_argument("--ragged", action="store_true",
                    help="only time the ragged serving step of the c3 workload (live lengths 50-100%% "
                         "of the capacities, new token stored) and print its figures as one JSON line")
    ap.add_argument("--paged", type=int, default=0, metavar="ROWS",
                    help="with --ragged or --chunk: the cache in pages of ROWS rows (a power "
                         "of two >= 64) at shuffled page ids, through slimkv_decode_attn_paged "
                         "or slimkv_decode_attn_chunk_paged")
    ap.add_argument("--chunk", type=int, default=0, metavar="Q",
                    help="only time the ragged serving step with Q query tokens per sequence "
                         "(slimkv_decode_attn_chunk) and print its figures as one JSON line")
    ap.add_argument("--alibi", action="store_true",
                    help="only time the step as an ALiBi backbone runs it (slimkv_decode_attn_alibi) "
                         "and print its figures as one JSON line")
    ap.add_argument("--calibrate", action="store_true",
                    help="only run a plain 1 GiB device copy (torch) and a 512 MiB read-only "
                         "reduction, for scaling hardware byte counters and as a read ceiling")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def layer_call_bytes(wl, layer, elem):
    """Algorithmic HBM bytes of one latent call: cache rows + bases + q + outputs."""
    r = wl.ranks[layer]
    units = wl.batch * wl.num_kv_heads
    cache = units * (wl.num_beacons * 2 * r + 2 * wl.raw_window * wl.head_dim) * elem
    bases = wl.num_kv_heads * wl.head_dim * 2 * r * elem
    q = wl.batch * wl.num_q_heads * wl.head_dim * elem
    out = wl.batch * wl.num_q_heads * (wl.head_dim + 1) * 4
    return cache, cache + bases + q + out


def measured_traffic(workload_name):
    """HBM bytes per launch of the attention kernel from the committed
    rocprofv3 PMC summary, or None if that measurement was taken on other
    kernel sources or another workload."""
    rec_path = pathlib.Path(ROOT) / "profiles" / "attention_kernel_c3_traffic.json"
    if not rec_path.exists():
        return None
    rec = json.loads(rec_path.read_text())
    h = hashlib.sha256()
    for f in sorted((pathlib.Path(ROOT) / "latent_decode_attention_amd" / "csrc").iterdir()):
        h.update(f.name.encode())
        h.update(f.read_bytes())
    if rec.get("source_sha256") != h.hexdigest() or rec.get("workload") != workload_name:
        return None
    return rec["traffic_bytes_per_launch"]


def attn_kernel_bytes(wl, layer, elem):
    """Algorithmic bytes one latent call must move: the cache rows, q, U_K,
    U_V, and the fp32 out and lse."""
    return layer_call_bytes(wl, layer, elem)[1]


def time_calls(fn, iters, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters  # ms


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the method's "
              "hot path runs on one GPU's share; see DESIGN.md on sharding)", file=sys.stderr)
        sys.exit(2)

    import torch

    import latent_decode_attention_amd as lda
    import synth

    dev = torch.device("cuda:0")
    if args.calibrate:
        calibrate(torch, dev)
        return
    wl = synth.get_workload(args.workload)
    elem = wl.elem_bytes
    log(f"workload {wl.name}: {wl.layers} layers, B={wl.batch}, generating inputs on the GPU")
    layers = [synth.make_layer(wl, layer, device=dev) for layer in range(wl.layers)]
    if args.ragged:
        print(json.dumps(ragged_step(lda, synth, torch, dev, wl, layers, args.steps,
                                     page_rows=args.paged)), flush=True)
        return
    if args.alibi:
        print(json.dumps(alibi_step(lda, synth, torch, dev, wl, layers, args.steps)), flush=True)
        return
    if args.chunk:
        print(json.dumps(chunk_step(lda, synth, torch, dev, wl, layers, args.steps, args.chunk,
                                    page_rows=args.paged)),
              flush=True)
        return
    probs = [lda.problem_from_tensors(x.q, x.U_K, x.C_K, x.K_raw, U_V=x.U_V,
                                      rope_theta=wl.rope_theta, num_kv_heads=wl.num_kv_heads,
                                      scale=wl.scale) for x in layers]
    ws_bytes = max(lda.slimkv_workspace_bytes(p, lda.SLIMKV_OP_LATENT) for p in probs)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    out, lse = lda.alloc_outputs(probs[0], dev)
    torch.cuda.synchronize()

    def step():
        for p, x in zip(probs, layers):
            lda.slimkv_decode_attn(p, x.q, x.q_pos, x.U_K, x.U_V, x.C_K, x.C_V, x.K_raw, x.V_raw,
                                   out, lse, ws)

    log(f"warmup {args.warmup} steps, timing {args.steps}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    run, launch = step, "eager launches"
    if not args.eager:
        # A decode step's calls have no host work between them; a serving loop
        # replays them as one captured graph.  The replay must reproduce the
        # eager step bit for bit (the library allocates and resets nothing
        # outside its kernels, so the captured launches are the whole step).
        ref_out, ref_lse = out.clone(), lse.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        out.zero_()
        lse.zero_()
        graph.replay()
        torch.cuda.synchronize()
        if not (torch.equal(out, ref_out) and torch.equal(lse, ref_lse)):
            raise RuntimeError("graph replay differs from the eager step")
        run, launch = graph.replay, f"one captured HIP graph per step ({wl.layers} calls)"
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        run()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / args.steps
    tokens_per_s = wl.batch / (ms_step * 1e-3)
    cache_step = sum(layer_call_bytes(wl, layer, elem)[0] for layer in range(wl.layers))
    total_step = sum(layer_call_bytes(wl, layer, elem)[1] for layer in range(wl.layers))
    step_gbps = total_step / (ms_step * 1e-3) / 1e9
    log(f"{ms_step:.3f} ms/step, {tokens_per_s:.0f} tokens/s, {step_gbps:.0f} GB/s "
        f"(wall {wall:.2f}s)")

    # Each latent call is one kernel launch, so the events around the timed
    # region divided by the launches give that kernel's average launch time,
    # the short gap between back-to-back launches included.
    launches = wl.layers * args.steps
    kern_us = ms_step * 1e3 / wl.layers
    kern_bytes = sum(attn_kernel_bytes(wl, layer, elem) for layer in range(wl.layers)) / wl.layers
    achieved = kern_bytes / (kern_us * 1e-6) / 1e9
    log(f"attention kernel: {kern_us:.1f} us average over {launches} launches, "
        f"{achieved:.0f} GB/s")

    result = {
        "metric": "decode-attn tokens/s + HBM GB/s (% peak) at 128K, latent vs full-KV, 1 GPU",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "fp32",
        "data": "synthetic (seeded Gaussian caches at the model's shapes, generated on the GPU)",
        "config": {
            "workload": (f"{wl.name}: decode attention over {wl.layers} layers, batch "
                         f"{wl.batch}, {wl.num_q_heads}/{wl.num_kv_heads} heads, d=128, "
                         f"{wl.context} context as {wl.num_beacons} beacons (ranks "
                         f"{min(wl.ranks)}-{max(wl.ranks)}, mean {sum(wl.ranks) / wl.layers:g}) "
                         f"+ {wl.raw_window} raw tokens"),
            "global_batch": wl.batch,
            "seq_len": wl.context,
            "layers": wl.layers,
            "parallelism": "single GPU",
            "launch": launch,
        },
        "hbm_gbps": round(step_gbps, 1),
        "hbm_frac_of_peak": round(step_gbps / HBM_PEAK_GBPS, 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(wl.name),
            "kernel": "attention_kernel (the whole latent call is this one launch)",
            "bytes_per_launch": int(kern_bytes),
            "launch_us": round(kern_us, 2),
            "launches_timed": launches,
        },
    }

    if not args.no_compare:
        result["comparison"] = compare(lda, synth, torch, dev)
        if args.workload == "c3":
            result["comparison"]["c3_ragged_step"] = ragged_step(lda, synth, torch, dev, wl, layers,
                                                                 args.steps)
            result["comparison"]["c3_paged_step"] = ragged_step(lda, synth, torch, dev, wl, layers,
                                                                args.steps, page_rows=64)
            result["comparison"]["c3_chunk4_step"] = chunk_step(lda, synth, torch, dev, wl, layers,
                                                                 args.steps, 4)
            result["comparison"]["c3_chunk4_paged_step"] = chunk_step(
                lda, synth, torch, dev, wl, layers, args.steps, 4, page_rows=64)
            result["comparison"]["c3_alibi_step"] = alibi_step(lda, synth, torch, dev, wl, layers,
                                                               args.steps)
            result["comparison"]["c4_step"] = other_step(lda, synth, torch, dev, "c4", args.steps)

    del ws
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, layers, args.cpu_budget_s, synth)
    print(json.dumps(result), flush=True)


def calibrate(torch, dev):
    """A plain copy of known size (1 GiB read + 1 GiB written per launch) to
    scale FETCH_SIZE / WRITE_SIZE counters, and a read-only sum over 512 MiB
    as a streaming-read reference."""
    n = 1 << 30
    src = torch.ones(n // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    t_copy = time_calls(lambda: dst.copy_(src), 10, 3, torch)
    rd = src[: (n // 4)]
    t_sum = time_calls(lambda: rd.sum(dtype=torch.float32), 10, 3, torch)
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n,
                      "copy_us": round(t_copy * 1e3, 1),
                      "copy_gbps": round(2 * n / (t_copy * 1e-3) / 1e9, 1),
                      "sum_bytes_read": n // 2, "sum_us": round(t_sum * 1e3, 1),
                      "sum_read_gbps": round((n // 2) / (t_sum * 1e-3) / 1e9, 1)}), flush=True)


def compare(lda, synth, torch, dev):
    """One 128K layer (B=16): latent at 16x vs reconstruct on the same beacons
    vs full-KV over 131072 tokens, plus the latent sweep at 4x/8x/32x."""
    res = {}
    full_wl = synth.get_workload("c5_full")
    log("comparison: generating full-KV cache (131072 tokens)")
    K, V = synth.make_full_kv(full_wl, 0, device=dev)
    base = synth.make_layer(full_wl, 0, device=dev, num_beacons=0, raw_window=128)
    pf = lda.make_problem(batch=full_wl.batch, num_q_heads=full_wl.num_q_heads,
                          num_kv_heads=full_wl.num_kv_heads, num_beacons=0, rank_k=0, rank_v=0,
                          raw_window=full_wl.context, scale=full_wl.scale,
                          rope_theta=full_wl.rope_theta, dtype=full_wl.dtype)
    out, lse = lda.alloc_outputs(pf, dev)
    ws = lda.alloc_workspace(pf, lda.SLIMKV_OP_FULL_KV, dev)
    t_full = time_calls(lambda: lda.full_kv_attn(pf, base.q, base.q_pos, K, V, out, lse, ws),
                        10, 3, torch)
    bytes_full = 2 * K.numel() * K.element_size()
    res["full_kv"] = {"us": round(t_full * 1e3, 1), "gbps": round(bytes_full / t_full / 1e6, 1)}
    del K, V, ws
    torch.cuda.empty_cache()
    for key in ("c5_4x", "c5_8x", "c5_16x", "c5_32x"):
        wl = synth.get_workload(key)
        x = synth.make_layer(wl, 0, device=dev)
        p = lda.problem_from_tensors(x.q, x.U_K, x.C_K, x.K_raw, U_V=x.U_V,
                                     rope_theta=wl.rope_theta, num_kv_heads=wl.num_kv_heads,
                                     scale=wl.scale)
        ws = lda.alloc_workspace(p, lda.SLIMKV_OP_LATENT, dev)
        t = time_calls(lambda: lda.slimkv_decode_attn(p, x.q, x.q_pos, x.U_K, x.U_V, x.C_K,
                                                      x.C_V, x.K_raw, x.V_raw, out, lse, ws),
                       20, 3, torch)
        cache = wl.layer_bytes(0)
        entry = {"us": round(t * 1e3, 1), "gbps": round(cache / t / 1e6, 1),
                 "speedup_vs_full_kv": round(t_full / t, 2)}
        if key == "c5_16x":
            wsr = lda.alloc_workspace(p, lda.SLIMKV_OP_RECONSTRUCT, dev)
            tr = time_calls(lambda: lda.slimkv_reconstruct_attn(
                p, x.q, x.q_pos, x.U_K, x.U_V, x.C_K, x.C_V, x.K_raw, x.V_raw, out, lse, wsr),
                10, 3, torch)
            entry["reconstruct_us"] = round(tr * 1e3, 1)
            entry["speedup_vs_reconstruct"] = round(tr / t, 2)
            # the variant the page times: rebuilt beacon keys rotated at their
            # positions (one beacon per s tokens, at the end of its span)
            s_tok = wl.context // wl.num_beacons
            bpos = ((torch.arange(wl.num_beacons, device=dev, dtype=torch.int64) + 1) * s_tok
                    - 1).to(torch.int32)
            trr = time_calls(lambda: lda.slimkv_reconstruct_rope_attn(
                p, x.q, x.q_pos, x.U_K, x.U_V, x.C_K, x.C_V, x.K_raw, x.V_raw, bpos, out, lse,
                wsr), 10, 3, torch)
            entry["reconstruct_rope_us"] = round(trr * 1e3, 1)
            entry["speedup_vs_reconstruct_rope"] = round(trr / t, 2)
            del wsr
        res[key] = entry
        del x, ws
        torch.cuda.empty_cache()
        log(f"comparison {key}: {entry}")
    return res


def replay_ms(torch, step, steps):
    """Capture ``step`` as one graph and time its replays (ms per step)."""
    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    return time_calls(graph.replay, steps, 3, torch)


def ragged_step(lda, synth, torch, dev, wl, layers, steps, page_rows=0):
    """The same 32-layer step as a serving step over a ragged batch: each
    sequence keeps a seeded number of live beacons (4096..8192) and raw rows
    (1024..2047) in the arrays, and every layer attends and stores the step's
    new token (slimkv_decode_attn_ragged).  page_rows > 0: the cache lies in
    pages of that many rows at seeded, shuffled page ids, and the step runs
    slimkv_decode_attn_paged on them.  Bytes: the live rows, the new token's
    key and value read and written, q, the bases, out and lse (the page
    tables add 4 bytes per page, left out)."""
    elem = wl.elem_bytes
    first = synth.make_step(wl, layers[0], device=dev, beacons=(0.5, 1.0), raw=(0.5, 1.0))
    steps_in, probs, bytes_step = [], [], 0
    nb = first.num_beacons.cpu().numpy().clip(0, wl.num_beacons)
    rw = first.raw_len.cpu().numpy().clip(0, wl.raw_window)
    for layer, x in enumerate(layers):
        st = synth.make_step(wl, x, device=dev)
        st.num_beacons, st.raw_len = first.num_beacons, first.raw_len  # lengths are per sequence
        steps_in.append(st)
        probs.append(lda.problem_from_tensors(x.q, x.U_K, x.C_K, x.K_raw, U_V=x.U_V,
                                              rope_theta=wl.rope_theta,
                                              num_kv_heads=wl.num_kv_heads, scale=wl.scale))
        r = wl.ranks[layer]
        rows = wl.num_kv_heads * (int(nb.sum()) * 2 * r + int(rw.sum()) * 2 * wl.head_dim)
        new_tok = wl.batch * wl.num_kv_heads * wl.head_dim * 2 * 2  # k, v read and stored
        bytes_step += ((rows + new_tok) * elem + wl.num_kv_heads * wl.head_dim * 2 * r * elem
                       + wl.batch * wl.num_q_heads * wl.head_dim * elem
                       + wl.batch * wl.num_q_heads * (wl.head_dim + 1) * 4)
    ws = torch.zeros(max(lda.slimkv_workspace_bytes(p, lda.SLIMKV_OP_LATENT_RAGGED) for p in probs),
                     dtype=torch.uint8, device=dev)
    out, lse = lda.alloc_outputs(probs[0], dev)

    if page_rows:
        paged = [synth.make_paged(x, st, page_rows=page_rows) for x, st in zip(layers, steps_in)]
        tables = [lda.make_pages(page_rows=page_rows, beacon_table=pc.beacon_table,
                                 raw_table=pc.raw_table, beacon_pages=pc.beacon_pages,
                                 raw_pages=pc.raw_pages) for pc in paged]

        def step():
            for p, x, st, pc, tb in zip(probs, layers, steps_in, paged, tables):
                lda.slimkv_decode_attn_paged(p, tb, x.q, x.q_pos, x.U_K, x.U_V, pc.C_K, pc.C_V,
                                             pc.K_raw, pc.V_raw, st.num_beacons, st.raw_len,
                                             st.k_new, st.v_new, out, lse, ws)
    else:
        def step():
            for p, x, st in zip(probs, layers, steps_in):
                lda.slimkv_decode_attn_ragged(p, x.q, x.q_pos, x.U_K, x.U_V, x.C_K, x.C_V,
                                              x.K_raw, x.V_raw, st.num_beacons, st.raw_len,
                                              st.k_new, st.v_new, out, lse, ws)

    ms = replay_ms(torch, step, steps)
    gbps = bytes_step / (ms * 1e-3) / 1e9
    res = {"ms_per_step": round(ms, 4), "us_per_layer": round(ms * 1e3 / wl.layers, 2),
           "tokens_per_s": round(wl.batch / (ms * 1e-3), 1), "gbps": round(gbps, 1),
           "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
           "live_rows": f"beacons {int(nb.min())}..{int(nb.max())} (mean {nb.mean():.0f}), raw "
                        f"{int(rw.min())}..{int(rw.max())} (mean {rw.mean():.0f}) + new token"}
    if page_rows:
        res["page_rows"] = page_rows
        del paged, tables
    log(f"{'paged' if page_rows else 'ragged'} step: {res}")
    del ws
    torch.cuda.empty_cache()
    return res


def chunk_step(lda, synth, torch, dev, wl, layers, steps, num_tokens, page_rows=0):
    """The ragged serving step of ragged_step with a chunk of num_tokens
    query tokens per sequence (e.g. drafted tokens checked in one pass):
    every layer attends each token over the live rows and the chunk's tokens
    up to it, and stores the tokens (slimkv_decode_attn_chunk).  page_rows >
    0: the cache lies in pages of that many rows at seeded, shuffled page
    ids (slimkv_decode_attn_chunk_paged).  Bytes: the live rows, the tokens'
    keys and values read and written, the queries, the bases, out and lse."""
    elem = wl.elem_bytes
    Q = num_tokens
    first = synth.make_step(wl, layers[0], device=dev, beacons=(0.5, 1.0), raw=(0.5, 1.0))
    nb = first.num_beacons.cpu().numpy().clip(0, wl.num_beacons)
    rw = first.raw_len.cpu().numpy().clip(0, wl.raw_window - Q)
    raw_len = torch.from_numpy(rw.astype("int32")).to(dev)
    chunks, probs, bytes_step = [], [], 0
    for layer, x in enumerate(layers):
        c = synth.make_chunk(wl, x, Q, device=dev)
        c.num_beacons, c.raw_len = first.num_beacons, raw_len  # lengths are per sequence
        chunks.append(c)
        probs.append(lda.problem_from_tensors(x.q, x.U_K, x.C_K, x.K_raw, U_V=x.U_V,
                                              rope_theta=wl.rope_theta,
                                              num_kv_heads=wl.num_kv_heads, scale=wl.scale))
        r = wl.ranks[layer]
        rows = wl.num_kv_heads * (int(nb.sum()) * 2 * r + int(rw.sum()) * 2 * wl.head_dim)
        new_tok = Q * wl.batch * wl.num_kv_heads * wl.head_dim * 2 * 2  # k, v read and stored
        bytes_step += ((rows + new_tok) * elem + wl.num_kv_heads * wl.head_dim * 2 * r * elem
                       + Q * wl.batch * wl.num_q_heads * wl.head_dim * elem
                       + Q * wl.batch * wl.num_q_heads * (wl.head_dim + 1) * 4)
    ws = torch.zeros(max(lda.slimkv_chunk_workspace_bytes(p, Q) for p in probs),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((wl.batch, Q, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((wl.batch, Q, wl.num_q_heads), dtype=torch.float32, device=dev)

    if page_rows:
        paged = [synth.make_paged(x, c, page_rows=page_rows) for x, c in zip(layers, chunks)]
        tables = [lda.make_pages(page_rows=page_rows, beacon_table=pc.beacon_table,
                                 raw_table=pc.raw_table, beacon_pages=pc.beacon_pages,
                                 raw_pages=pc.raw_pages) for pc in paged]

        def step():
            for p, x, c, pc, tb in zip(probs, layers, chunks, paged, tables):
                lda.slimkv_decode_attn_chunk_paged(p, tb, Q, c.q, x.q_pos, x.U_K, x.U_V, pc.C_K,
                                                   pc.C_V, pc.K_raw, pc.V_raw, c.num_beacons,
                                                   c.raw_len, c.k_new, c.v_new, out, lse, ws)
    else:
        def step():
            for p, x, c in zip(probs, layers, chunks):
                lda.slimkv_decode_attn_chunk(p, Q, c.q, x.q_pos, x.U_K, x.U_V, x.C_K, x.C_V,
                                             x.K_raw, x.V_raw, c.num_beacons, c.raw_len, c.k_new,
                                             c.v_new, out, lse, ws)

    ms = replay_ms(torch, step, steps)
    gbps = bytes_step / (ms * 1e-3) / 1e9
    res = {"tokens_per_chunk": Q, "ms_per_step": round(ms, 4),
           "us_per_layer": round(ms * 1e3 / wl.layers, 2),
           "query_tokens_per_s": round(wl.batch * Q / (ms * 1e-3), 1), "gbps": round(gbps, 1),
           "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
           "live_rows": f"beacons {int(nb.min())}..{int(nb.max())} (mean {nb.mean():.0f}), raw "
                        f"{int(rw.min())}..{int(rw.max())} (mean {rw.mean():.0f}) + {Q} tokens"}
    if page_rows:
        res["page_rows"] = page_rows
        del paged, tables
    log(f"{'paged ' if page_rows else ''}chunk step: {res}")
    del ws, chunks
    torch.cuda.empty_cache()
    return res


def alibi_step(lda, synth, torch, dev, wl, layers, steps):
    """The same 32-layer step as an ALiBi backbone would run it
    (slimkv_decode_attn_alibi: no rotation, the ALiBi paper's slopes, one
    beacon per 16 tokens).  Bytes as for the headline step."""
    import numpy as np
    elem = wl.elem_bytes
    probs = [lda.problem_from_tensors(x.q, x.U_K, x.C_K, x.K_raw, U_V=x.U_V,
                                      rope_theta=wl.rope_theta, num_kv_heads=wl.num_kv_heads,
                                      scale=wl.scale) for x in layers]
    ws = torch.zeros(max(lda.slimkv_workspace_bytes(p, lda.SLIMKV_OP_LATENT) for p in probs),
                     dtype=torch.uint8, device=dev)
    out, lse = lda.alloc_outputs(probs[0], dev)
    slopes = torch.as_tensor(synth.alibi_slopes(wl.num_q_heads).astype(np.float32), device=dev)
    first, stride = synth.beacon_grid(16)

    def step():
        for p, x in zip(probs, layers):
            lda.slimkv_decode_attn_alibi(p, x.q, x.q_pos, x.U_K, x.U_V, x.C_K, x.C_V, x.K_raw,
                                         x.V_raw, slopes, first, stride, out, lse, ws)

    ms = replay_ms(torch, step, steps)
    total = sum(layer_call_bytes(wl, layer, elem)[1] for layer in range(wl.layers))
    gbps = total / (ms * 1e-3) / 1e9
    res = {"ms_per_step": round(ms, 4), "us_per_layer": round(ms * 1e3 / wl.layers, 2),
           "tokens_per_s": round(wl.batch / (ms * 1e-3), 1), "gbps": round(gbps, 1),
           "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    log(f"alibi step: {res}")
    del ws
    torch.cuda.empty_cache()
    return res


def other_step(lda, synth, torch, dev, name, steps):
    """Another workload's full decode step (every layer), replayed as a graph."""
    wl = synth.get_workload(name)
    elem = wl.elem_bytes
    log(f"{name}: generating {wl.layers} layers")
    layers = [synth.make_layer(wl, layer, device=dev) for layer in range(wl.layers)]
    probs = [lda.problem_from_tensors(x.q, x.U_K, x.C_K, x.K_raw, U_V=x.U_V,
                                      rope_theta=wl.rope_theta, num_kv_heads=wl.num_kv_heads,
                                      scale=wl.scale) for x in layers]
    ws = torch.zeros(max(lda.slimkv_workspace_bytes(p, lda.SLIMKV_OP_LATENT) for p in probs),
                     dtype=torch.uint8, device=dev)
    out, lse = lda.alloc_outputs(probs[0], dev)

    def step():
        for p, x in zip(probs, layers):
            lda.slimkv_decode_attn(p, x.q, x.q_pos, x.U_K, x.U_V, x.C_K, x.C_V, x.K_raw, x.V_raw,
                                   out, lse, ws)

    ms = replay_ms(torch, step, steps)
    total = sum(layer_call_bytes(wl, layer, elem)[1] for layer in range(wl.layers))
    gbps = total / (ms * 1e-3) / 1e9
    res = {"ms_per_step": round(ms, 4), "us_per_layer": round(ms * 1e3 / wl.layers, 2),
           "tokens_per_s": round(wl.batch / (ms * 1e-3), 1), "gbps": round(gbps, 1),
           "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    log(f"{name} step: {res}")
    del layers, ws
    torch.cuda.empty_cache()
    return res


def cpu_baseline(wl, layers, budget_s, synth):
    """The fp64 oracle on this host's cores over whole layers (the same
    inputs the GPU ran, copied to host memory once), in passes over the
    step's layers until the time budget is spent; the step time is the time
    per multiply-add times the step's multiply-add count (each layer's count
    depends on its rank)."""
    import oracle

    threads = oracle.max_threads()

    def macs(layer):
        r = wl.ranks[layer]
        per_head = wl.num_beacons * 2 * r + 2 * wl.raw_window * wl.head_dim + 2 * wl.head_dim * r
        return wl.batch * wl.num_q_heads * per_head

    st = synth.to_numpy_storage
    host = {}
    done, spent, calls = 0, 0.0, 0
    while spent < budget_s and calls < 64 * wl.layers:
        layer = calls % wl.layers
        if layer not in host:
            x = layers[layer]
            host[layer] = [st(t) for t in (x.q, x.q_pos, x.U_K, x.U_V, x.C_K, x.C_V, x.K_raw,
                                           x.V_raw)]
        t0 = time.perf_counter()
        oracle.decode(*host[layer], num_kv_heads=wl.num_kv_heads, scale=wl.scale,
                      rope_theta=wl.rope_theta, threads=threads)
        spent += time.perf_counter() - t0
        done += macs(layer)
        calls += 1
    log(f"cpu oracle: {calls} layer calls in {spent:.1f}s")
    total = sum(macs(layer) for layer in range(wl.layers))
    step_s = spent * total / done
    passes = f"{calls / wl.layers:.2f} passes over the {wl.layers} layers"
    return {"value": round(wl.batch / step_s, 3), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"{calls} layer calls ({passes}; all {wl.batch * wl.num_kv_heads} units "
                       f"each) timed in {spent:.1f}s with fp64 C+OpenMP; step time {step_s:.2f}s "
                       f"= time per multiply-add x the step's multiply-add count")}


if __name__ == "__main__":
    main()
