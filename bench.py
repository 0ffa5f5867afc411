#!/usr/bin/env python3
"""Decode-attention benchmark for libslimkv on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3]
                    [--no-cpu-baseline] [--no-compare] [--launched]

A step is one decode token's attention over every layer of the workload:
for the default workload (Llama-3.1-8B shape, 128K context, 16x token
compression, batch 16) that is 32 calls of slimkv_decode_attn, one per
layer, each with its own latent rank.  All inputs are generated on the GPU
before timing and stay resident in HBM.  The step's calls are captured once
as a HIP graph and replayed, as a serving loop does to keep host overhead
off the GPU's timeline (checked bit for bit against the same calls launched
directly; --launched times those instead, and the other form is reported
beside the headline).  Launched from Python, the calls are within 1-2% of
the replays on a quiet host and up to 4% slower on a busy one.  The timed region is bracketed by device
synchronisation and measured with events on the stream the library
launches on, one event between consecutive steps, so the line carries the
mean over the region and the median / p10 / p90 of the single steps.
Prints ONE JSON line.

Reported beside the headline tokens/s:
  * roofline of the sweep kernel: algorithmic bytes per launch over its
    average launch time from the events (gaps between launches included),
    against 8 TB/s; the same figure from the committed rocprofv3
    kernel-trace summary when it was taken on these kernel sources; and the
    streaming-read ceiling, a plain read of the same bytes by the library's
    own read kernel (slimkv_bench_stream_read) in the same process;
  * the comparison at 128K on one layer: latent path at 4/8/16/32x vs the
    reconstruct-then-attend paths on the same beacons (without and with the
    rotation of rebuilt beacon keys) and vs uncompressed full-KV attention
    over all 131072 tokens; the 32K one-layer workload; the ragged serving
    step, over capacity-sized arrays and over a paged cache, and with 4
    query tokens per sequence; the step as an ALiBi backbone runs it; the
    48-layer Qwen step.  One-layer calls rotate over copies of their inputs
    that together exceed 1 GB, so no call finds its inputs in the 256 MB
    last-level cache;
  * the fp64 CPU oracle timed on a bounded sample on this host's cores; its
    first layer is the step's last one, whose outputs the GPU left in
    out/lse after the timed replays, so the same run checks what it timed
    against the oracle (the "parity" block).

    python bench.py --calibrate        plain copy / read / write kernels of
                                       known size, for scaling PMC counters
    python bench.py --profile-summary DIR
                                       summarise a rocprofv3 kernel trace
                                       (CSV in DIR) per kernel instance
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import pathlib
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
ROTATE_BYTES = 1_100_000_000  # one-layer calls rotate over input copies totalling more


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--launched", action="store_true",
                    help="time the step's calls launched directly instead of one captured HIP "
                         "graph per step (both are always checked bit for bit against each other, "
                         "and the other one is reported beside the headline)")
    ap.add_argument("--ragged", action="store_true",
                    help="only time the ragged serving step of the c3 workload (live lengths 50-100%% "
                         "of the capacities, new token stored) and print its figures as one JSON line")
    ap.add_argument("--even-lengths", action="store_true",
                    help="with --ragged or --chunk: every sequence at the drawn lengths' means (the "
                         "same live bytes, split evenly over the units)")
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
    ap.add_argument("--only", default="",
                    help="only time one comparison entry (c2, c5_4x, c5_8x, c5_16x, c5_32x, "
                         "full_kv, read_ceiling) and print it as one JSON line")
    ap.add_argument("--calibrate", action="store_true",
                    help="only run plain kernels of known size (a 1 GiB copy, a 1 GiB read, a "
                         "1 GiB write) for scaling hardware byte counters")
    ap.add_argument("--report", nargs="+", metavar="JSON", default=None,
                    help="print a markdown report of benchmark results: files holding one bench "
                         "JSON line each, or a driver record with the line under 'parsed' (no GPU "
                         "needed)")
    ap.add_argument("--profile-summary", metavar="DIR", default="",
                    help="summarise the rocprofv3 kernel trace (*kernel_trace.csv) under DIR and "
                         "print it as JSON (no GPU needed): the attention kernel's dispatches "
                         "in the headline's timed steps of a bench run of --workload with the "
                         "same --steps, per layer and per step")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE"),
                    default=None,
                    help="summarise rocprofv3 --pmc runs (*counter_collection.csv under each "
                         "directory): FETCH_SIZE and WRITE_SIZE of a bench run of --workload "
                         "with the same --steps, and of 'bench.py --calibrate', which gives the "
                         "scale from counter units to bytes (no GPU needed)")
    ap.add_argument("--kernel", default="attention_kernel",
                    help="with --profile-summary or --traffic-summary: the kernel to summarise; "
                         "other than attention_kernel, every dispatch of it, per instance")
    ap.add_argument("--record", metavar="NAME", default="",
                    help="with --profile-summary or --traffic-summary: also write "
                         "profiles/NAME.json (read by the bench for the same kernel sources) "
                         "and profiles/NAME.md")
    ap.add_argument("--run-json", nargs="+", metavar="JSON", default=[],
                    help="with --profile-summary (one file) or --traffic-summary (two: the FETCH "
                         "and the WRITE run): the JSON line each profiled bench run printed, for "
                         "its warm-up step counts")
    ap.add_argument("--algorithmic-bytes", type=float, default=0.0,
                    help="with --traffic-summary --kernel K --record: the bytes one dispatch of K "
                         "must move, for the measured / algorithmic ratio")
    ap.add_argument("--label", default="",
                    help="with --record and --kernel other than attention_kernel: the run's "
                         "workload, in words")
    ap.add_argument("--untraced", metavar="JSON", default="",
                    help="with --record: the bench JSON line of the same command run without "
                         "the profiler on the same box, quoted beside the trace")
    ap.add_argument("--command", metavar="TEXT", nargs="+", default=None,
                    help="with --record: the commands that made the profile, for the summary")
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


def source_sha256():
    """sha256 over the kernel sources (name and bytes of every file under csrc/)."""
    h = hashlib.sha256()
    for f in sorted((pathlib.Path(ROOT) / "latent_decode_attention_amd" / "csrc").iterdir()):
        h.update(f.name.encode())
        h.update(f.read_bytes())
    return h.hexdigest()


def committed_record(name, workload_name):
    """A committed summary under profiles/ (JSON), or None if it was taken on
    other kernel sources or another workload."""
    rec_path = pathlib.Path(ROOT) / "profiles" / name
    if not rec_path.exists():
        return None
    rec = json.loads(rec_path.read_text())
    if rec.get("source_sha256") != source_sha256() or rec.get("workload") != workload_name:
        return None
    return rec


def pct(xs):
    """(median, p10, p90) of a list, in its units."""
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    p10, p50, p90 = np.percentile(a, [10, 50, 90])
    return float(p50), float(p10), float(p90)


WARM_MIN_S = 0.1  # untimed warm-up before every timed region lasts at least this long


def timed_steps(torch, run, steps, warmup, info=None):
    """Run ``run`` warmup times -- and on, in groups of 4, until the warm-up
    has lasted WARM_MIN_S of wall time -- then ``steps`` times back to back
    with an event recorded before the first and after every step, all on the
    current stream.  Returns (mean ms over the whole region, per-step ms).

    The floor on the warm-up's length: after the GPU has been idle (input
    generation, graph capture, host work between measurements) its first
    ~15 ms of streaming run up to 15% slower (kernel traces of the c3 step
    show ~6 slow steps after an idle gap, whichever launch form), so a
    fixed count of short warm-up steps would leave part of that ramp inside
    the timed region.  info (a dict): receives the warm-up steps run."""
    t0 = time.perf_counter()
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    n = warmup
    while time.perf_counter() - t0 < WARM_MIN_S:
        for _ in range(4):
            run()
        n += 4
        torch.cuda.synchronize()
    if info is not None:
        info["warmup_steps"] = n
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        run()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return evs[0].elapsed_time(evs[-1]) / steps, per


RELEASE_SETTLE_S = 1.0  # wait after returning freed device memory to the driver


def release(torch):
    """Return the caching allocator's free blocks to the driver, then wait
    RELEASE_SETTLE_S before anything else is timed.  For about half a
    second after a large release, HBM-bound kernels run slower: the c3 step
    ran at 73.8 instead of 70.6 us per layer for ~0.45 s after the paged
    step's 16 GiB of page pools were released, and at 70.6 while the same
    blocks stayed in torch's cache (the release call itself returned in
    ~30 ms)."""
    torch.cuda.empty_cache()
    torch.cuda.synchronize()
    time.sleep(RELEASE_SETTLE_S)


def capture(torch, fn):
    """Run ``fn`` once eagerly, then capture it as a HIP graph."""
    fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    return graph


def step_stats(ms, per):
    med, p10, p90 = pct(per)
    return {"ms_per_step": round(ms, 4), "median_ms": round(med, 4), "p10_ms": round(p10, 4),
            "p90_ms": round(p90, 4)}


def main():
    args = parse_args()
    if args.report:
        print(report(args.report), end="")
        return
    if args.profile_summary or args.traffic_summary:
        import synth
        wl = synth.get_workload(args.workload)
        if args.kernel != "attention_kernel":
            summ = (instance_trace_summary(args.profile_summary, args.kernel) if args.profile_summary
                    else instance_traffic_summary(*args.traffic_summary, args.kernel))
        elif args.profile_summary:
            summ = profile_summary(args.profile_summary, wl, args.steps, other_warm(args.run_json, 0))
        else:
            summ = traffic_summary(*args.traffic_summary, wl, args.steps,
                                   (other_warm(args.run_json, 0), other_warm(args.run_json, 1)))
        if args.record:
            write_record(args.record, summ, args)
        print(json.dumps(summ), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: this build runs "
              "the attention on one GPU's share only (sharding by KV head or batch needs no "
              "exchange and is described in the design notes, not built)", file=sys.stderr)
        sys.exit(2)

    import torch

    import latent_decode_attention_amd as lda
    import synth

    dev = torch.device("cuda:0")
    if args.calibrate:
        calibrate(lda, torch, dev)
        return
    if args.only:
        print(json.dumps(compare(lda, synth, torch, dev, only=args.only)), flush=True)
        return
    wl = synth.get_workload(args.workload)
    elem = wl.elem_bytes
    log(f"workload {wl.name}: {wl.layers} layers, B={wl.batch}, generating inputs on the GPU")
    layers = [synth.make_layer(wl, layer, device=dev) for layer in range(wl.layers)]
    if args.ragged:
        print(json.dumps(ragged_step(lda, synth, torch, dev, wl, layers, args.steps,
                                     page_rows=args.paged, even=args.even_lengths)), flush=True)
        return
    if args.alibi:
        print(json.dumps(alibi_step(lda, synth, torch, dev, wl, layers, args.steps)), flush=True)
        return
    if args.chunk:
        print(json.dumps(chunk_step(lda, synth, torch, dev, wl, layers, args.steps, args.chunk,
                                    page_rows=args.paged, even=args.even_lengths)),
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

    log(f"warmup {args.warmup} steps (and at least {WARM_MIN_S * 1e3:.0f} ms), timing {args.steps}")
    step()
    torch.cuda.synchronize()
    # The step's calls have no host work between them: they are launched
    # back to back on one stream (what a native serving loop does), or
    # replayed as one captured graph (what a Python serving loop does to save
    # launch overhead).  The replay must reproduce the launched step bit for
    # bit: the library allocates and resets nothing outside its kernels, so
    # the captured launches are the whole step.
    ref_out, ref_lse = out.clone(), lse.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    out.zero_()
    lse.zero_()
    graph.replay()
    torch.cuda.synchronize()
    if not (torch.equal(out, ref_out) and torch.equal(lse, ref_lse)):
        raise RuntimeError("graph replay differs from the launched step")
    modes = {"launched": (step, f"{wl.layers} calls launched back to back on one stream"),
             "graph": (graph.replay, f"one captured HIP graph per step ({wl.layers} calls)")}
    head, other = ("launched", "graph") if args.launched else ("graph", "launched")
    run, launch = modes[head]
    t0 = time.perf_counter()
    warm_head, warm_other = {}, {}
    ms_step, per_step = timed_steps(torch, run, args.steps, args.warmup, warm_head)
    wall = time.perf_counter() - t0
    ms_other, per_other = timed_steps(torch, modes[other][0], args.steps, 2, warm_other)
    tokens_per_s = wl.batch / (ms_step * 1e-3)
    total_step = sum(layer_call_bytes(wl, layer, elem)[1] for layer in range(wl.layers))
    step_gbps = total_step / (ms_step * 1e-3) / 1e9
    stats = step_stats(ms_step, per_step)
    log(f"{ms_step:.4f} ms/step (median {stats['median_ms']}, p10 {stats['p10_ms']}, p90 "
        f"{stats['p90_ms']}), {tokens_per_s:.0f} tokens/s, {step_gbps:.0f} GB/s (wall {wall:.2f}s)")

    # Each latent call is one kernel launch, so the events around the timed
    # region divided by the launches give that kernel's average launch time,
    # the short gap between back-to-back launches included.
    launches = wl.layers * args.steps
    kern_us = ms_step * 1e3 / wl.layers
    kern_bytes = sum(layer_call_bytes(wl, layer, elem)[1] for layer in range(wl.layers)) / wl.layers
    achieved = kern_bytes / (kern_us * 1e-6) / 1e9
    log(f"attention kernel: {kern_us:.2f} us average over {launches} launches, "
        f"{achieved:.0f} GB/s ({achieved / HBM_PEAK_GBPS:.4f} of peak)")
    traffic = committed_record(f"attention_kernel_{args.workload}_traffic.json", wl.name)
    prof = committed_record(f"attention_kernel_{args.workload}_trace.json", wl.name)
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": traffic["traffic_bytes_per_launch"] if traffic else None,
        "kernel": "attention_kernel (the whole latent call is this one launch)",
        "bytes_per_launch": int(kern_bytes),
        "launch_us": round(kern_us, 2),
        "launch_us_from": "events over the timed region / launches (gaps included); frac uses it",
        "launches_timed": launches,
        "rocprof": ({"launch_us": prof["launch_us"], "frac": prof["frac"],
                     "summary": prof["summary"], "traced_step_ms": prof.get("traced_step_ms")}
                    if prof else None),
    }
    other_stats = step_stats(ms_other, per_other)
    other_stats.update({"tokens_per_s": round(wl.batch / (ms_other * 1e-3), 1),
                        "launch_us": round(ms_other * 1e3 / wl.layers, 2), "launch": modes[other][1]})
    log(f"same step, {other}: {other_stats}")
    result = {
        "metric": "decode-attn tokens/s + HBM GB/s (% peak) at 128K, latent vs full-KV, 1 GPU",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": {"headline": warm_head["warmup_steps"], "other": warm_other["warmup_steps"],
                             "floor_ms": WARM_MIN_S * 1e3},
        "ms_per_step": round(ms_step, 4),
        "median_ms_per_step": stats["median_ms"],
        "p10_ms_per_step": stats["p10_ms"],
        "p90_ms_per_step": stats["p90_ms"],
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
        "roofline": roofline,
        f"step_{other}": other_stats,
    }
    # the last layer's out / lse, as the timed replays left them (checked
    # against the oracle in the CPU-baseline leg)
    last_out, last_lse = out.double().cpu().numpy(), lse.double().cpu().numpy()

    ceiling = read_ceiling(lda, torch, dev, int(kern_bytes))
    roofline["read_ceiling"] = ceiling
    log(f"read ceiling: {ceiling}")

    if not args.no_compare:
        result["comparison"] = compare(lda, synth, torch, dev)
        if args.workload == "c3":
            result["comparison"]["c3_ragged_step"] = ragged_step(lda, synth, torch, dev, wl, layers,
                                                                 args.steps)
            result["comparison"]["c3_paged_step"] = ragged_step(lda, synth, torch, dev, wl, layers,
                                                                args.steps, page_rows=64)
            # the same live bytes with every sequence at the mean lengths: what
            # an even split of the work over the workgroups gives
            result["comparison"]["c3_ragged_step_even_lengths"] = ragged_step(
                lda, synth, torch, dev, wl, layers, args.steps, even=True)
            result["comparison"]["c3_chunk4_step"] = chunk_step(lda, synth, torch, dev, wl, layers,
                                                                 args.steps, 4)
            result["comparison"]["c3_chunk4_paged_step"] = chunk_step(
                lda, synth, torch, dev, wl, layers, args.steps, 4, page_rows=64)
            result["comparison"]["c3_chunk4_step_even_lengths"] = chunk_step(
                lda, synth, torch, dev, wl, layers, args.steps, 4, even=True)
            result["comparison"]["c3_alibi_step"] = alibi_step(lda, synth, torch, dev, wl, layers,
                                                               args.steps)
            result["comparison"]["c4_step"] = other_step(lda, synth, torch, dev, "c4", args.steps)

    del ws
    release(torch)
    if not args.no_cpu_baseline:
        base, parity = cpu_baseline(wl, layers, args.cpu_budget_s, synth, last_out, last_lse)
        result["cpu_baseline"] = base
        result["parity"] = parity
    else:
        result["parity"] = None
    print(json.dumps(result), flush=True)


# ---------------------------------------------------------------------------
# Plain kernels: the streaming-read ceiling and counter calibration.

def read_ceiling(lda, torch, dev, nbytes):
    """The fastest plain streaming read of ``nbytes`` bytes in one launch of
    the library's read kernel, over a sweep of its loads in flight per lane
    and grid sizes.  Two buffers alternate, each larger than half the
    last-level cache and together more than it, so no launch reads cached
    bytes.  Per configuration: a captured graph of 8 launches, replayed 5
    times; the per-launch time is the median replay / 8."""
    nbytes = (max(nbytes, 16) + 15) // 16 * 16
    bufs = [torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    best = None
    sweep = []
    for wgs in (cus, 2 * cus, 4 * cus, 8 * cus):
        for fl in (1, 2, 4, 8, 16):
            def fn():
                for i in range(8):
                    lda.slimkv_bench_stream_read(bufs[i % 2], sink, in_flight=fl, workgroups=wgs)
            g = capture(torch, fn)
            _, per = timed_steps(torch, g.replay, 5, 1)
            us = pct(per)[0] * 1e3 / 8
            sweep.append((wgs, fl, round(us, 2)))
            if best is None or us < best[0]:
                best = (us, wgs, fl)
            del g
    log("read sweep (workgroups, loads in flight per lane, us): " + str(sweep))
    us, wgs, fl = best
    gbps = nbytes / (us * 1e-6) / 1e9
    del bufs
    release(torch)
    return {"bytes": nbytes, "us": round(us, 2), "gbps": round(gbps, 1),
            "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "config": f"{wgs} workgroups x 256 threads, {fl} 16-byte loads in flight per lane",
            "kernel": "slimkv_bench_stream_read (libslimkv)"}


def calibrate(lda, torch, dev):
    """Plain kernels of known size, for scaling FETCH_SIZE / WRITE_SIZE: a
    1 GiB device copy (torch), a 1 GiB read (the library's read kernel) and
    a 1 GiB write (the library's flush kernel), three launches each."""
    n = 1 << 30
    src = torch.ones(n // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def t3(fn):
        fn()
        torch.cuda.synchronize()
        _, per = timed_steps(torch, fn, 3, 0)
        return pct(per)[0]

    rd = src[: (n // 2 - 8)]  # the read kernel takes at most 2^31 - 16 bytes: read 1 GiB - 16
    t_copy = t3(lambda: dst.copy_(src))
    t_read = t3(lambda: lda.slimkv_bench_stream_read(rd, sink, in_flight=4))
    t_write = t3(lambda: lda.slimkv_bench_flush(dst))
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n,
                      "copy_us": round(t_copy * 1e3, 1),
                      "read_bytes": rd.numel() * 2, "read_us": round(t_read * 1e3, 1),
                      "write_bytes": n, "write_us": round(t_write * 1e3, 1)}), flush=True)


# ---------------------------------------------------------------------------
# One-layer comparisons at 128K, with rotated inputs.

def rotated_call_us(torch, calls, reps=10):
    """Capture the list of calls (each over its own copy of the inputs) as
    one graph, replay it ``reps`` times with an event between replays, and
    return per-call (mean, median, p10, p90) in us."""
    def fn():
        for c in calls:
            c()
    g = capture(torch, fn)
    ms, per = timed_steps(torch, g.replay, reps, 2)
    n = len(calls)
    med, p10, p90 = pct(per)
    return ms * 1e3 / n, med * 1e3 / n, p10 * 1e3 / n, p90 * 1e3 / n


def timing_entry(us_tuple, nbytes):
    mean, med, p10, p90 = us_tuple
    gbps = nbytes / (mean * 1e-6) / 1e9
    return {"us": round(mean, 1), "median_us": round(med, 1), "p10_us": round(p10, 1),
            "p90_us": round(p90, 1), "gbps": round(gbps, 1),
            "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}


def layer_sets(synth, wl, dev, nbytes):
    """Copies of one layer's inputs (distinct seeds) that together exceed
    ROTATE_BYTES."""
    n = max(1, math.ceil(ROTATE_BYTES / nbytes))
    return [synth.make_layer(wl, 0, base_seed=s, device=dev) for s in range(n)]


def latent_bytes(wl):
    return layer_call_bytes(wl, 0, wl.elem_bytes)[1]


def recon_bytes(wl):
    """Reconstruct-then-attend: the latent bytes, plus the rebuilt beacon
    keys and values written once and read back once at full width."""
    units = wl.batch * wl.num_kv_heads
    return latent_bytes(wl) + 2 * 2 * units * wl.num_beacons * wl.head_dim * wl.elem_bytes


def compare(lda, synth, torch, dev, only=""):
    """One layer at 128K (B=16): the latent path at 4/8/16/32x vs the
    reconstruct paths on the same beacons (16x) vs full KV over 131072
    tokens; the 32K one-layer workload; the read ceiling on full KV's bytes."""
    res = {}
    keys = [only] if only else ["full_kv", "c5_4x", "c5_8x", "c5_16x", "c5_32x", "c2"]
    t_full = None
    if "full_kv" in keys or not only:
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
        bytes_full = 2 * K.numel() * K.element_size()
        us = rotated_call_us(torch, [lambda: lda.full_kv_attn(pf, base.q, base.q_pos, K, V, out,
                                                              lse, ws)], reps=10)
        t_full = us[0]
        res["full_kv"] = timing_entry(us, bytes_full)
        log(f"comparison full_kv: {res['full_kv']}")
        del K, V, ws
        release(torch)
    if only == "read_ceiling":
        return read_ceiling(lda, torch, dev, 403_310_592)
    for key in [k for k in keys if k.startswith("c5_") or k == "c2"]:
        wl = synth.get_workload(key)
        nbytes = latent_bytes(wl)
        sets = layer_sets(synth, wl, dev, nbytes)
        x0 = sets[0]
        p = lda.problem_from_tensors(x0.q, x0.U_K, x0.C_K, x0.K_raw, U_V=x0.U_V,
                                     rope_theta=wl.rope_theta, num_kv_heads=wl.num_kv_heads,
                                     scale=wl.scale)
        out, lse = lda.alloc_outputs(p, dev)
        ws = lda.alloc_workspace(p, lda.SLIMKV_OP_LATENT, dev)
        calls = [lambda x=x: lda.slimkv_decode_attn(p, x.q, x.q_pos, x.U_K, x.U_V, x.C_K, x.C_V,
                                                    x.K_raw, x.V_raw, out, lse, ws) for x in sets]
        entry = timing_entry(rotated_call_us(torch, calls, reps=10), nbytes)
        entry["input_copies"] = len(sets)
        if t_full is not None and key != "c2":
            entry["speedup_vs_full_kv"] = round(t_full / entry["us"], 2)
        if key == "c2":
            entry["tokens_per_s"] = round(wl.batch / (entry["us"] * 1e-6), 1)
        if key == "c5_16x":
            del ws
            release(torch)
            rb = recon_bytes(wl)
            rsets = sets[: max(1, math.ceil(ROTATE_BYTES / rb))]
            wsr = lda.alloc_workspace(p, lda.SLIMKV_OP_RECONSTRUCT, dev)
            rcalls = [lambda x=x: lda.slimkv_reconstruct_attn(
                p, x.q, x.q_pos, x.U_K, x.U_V, x.C_K, x.C_V, x.K_raw, x.V_raw, out, lse, wsr)
                for x in rsets]
            er = timing_entry(rotated_call_us(torch, rcalls, reps=10), rb)
            entry["reconstruct"] = er
            entry["speedup_vs_reconstruct"] = round(er["us"] / entry["us"], 2)
            # the variant the page times: rebuilt beacon keys rotated at their
            # positions (one beacon per s tokens, at the end of its span)
            s_tok = wl.context // wl.num_beacons
            bpos = ((torch.arange(wl.num_beacons, device=dev, dtype=torch.int64) + 1) * s_tok
                    - 1).to(torch.int32)
            rrcalls = [lambda x=x: lda.slimkv_reconstruct_rope_attn(
                p, x.q, x.q_pos, x.U_K, x.U_V, x.C_K, x.C_V, x.K_raw, x.V_raw, bpos, out, lse,
                wsr) for x in rsets]
            err = timing_entry(rotated_call_us(torch, rrcalls, reps=10), rb)
            entry["reconstruct_rope"] = err
            entry["speedup_vs_reconstruct_rope"] = round(err["us"] / entry["us"], 2)
            del wsr
        res[key] = entry
        del sets, x0, calls
        release(torch)
        log(f"comparison {key}: {entry}")
    return res if not only else res.get(only, res)


# ---------------------------------------------------------------------------
# Whole steps of other entry points and workloads, replayed as graphs.

def replay_stats(torch, step, steps):
    """Capture ``step`` as one graph and time its replays."""
    g = capture(torch, step)
    return timed_steps(torch, g.replay, steps, 3)


def even_lengths(synth, wl, layer, dev, first):
    """The step's lengths with every sequence at the drawn lengths' (rounded)
    means: about the same live bytes, split evenly over the units, so that
    the schedule's pieces all carry the same tiles."""
    m = (int(round(float(first.num_beacons.float().mean()))),
         int(round(float(first.raw_len.float().mean()))))
    return synth.make_step(wl, layer, device=dev, fixed={b: m for b in range(wl.batch)})


def ragged_step(lda, synth, torch, dev, wl, layers, steps, page_rows=0, even=False):
    """The same 32-layer step as a serving step over a ragged batch: each
    sequence keeps a seeded number of live beacons (4096..8192) and raw rows
    (1024..2047) in the arrays, and every layer attends and stores the step's
    new token (slimkv_decode_attn_ragged).  page_rows > 0: the cache lies in
    pages of that many rows at seeded, shuffled page ids, and the step runs
    slimkv_decode_attn_paged on them.  Bytes: the live rows, the new token's
    key and value read and written, q, the bases, out and lse (the page
    tables add 4 bytes per page, left out).  even: every sequence at the
    drawn lengths' means instead (even_lengths)."""
    elem = wl.elem_bytes
    first = synth.make_step(wl, layers[0], device=dev, beacons=(0.5, 1.0), raw=(0.5, 1.0))
    if even:
        first = even_lengths(synth, wl, layers[0], dev, first)
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
        # the call stores the new token into the raw arrays: give it copies,
        # so the headline step's inputs (checked against the oracle at the
        # end) stay as they were
        raws = [(x.K_raw.clone(), x.V_raw.clone()) for x in layers]

        def step():
            for p, x, st, (kr, vr) in zip(probs, layers, steps_in, raws):
                lda.slimkv_decode_attn_ragged(p, x.q, x.q_pos, x.U_K, x.U_V, x.C_K, x.C_V,
                                              kr, vr, st.num_beacons, st.raw_len,
                                              st.k_new, st.v_new, out, lse, ws)

    ms, per = replay_stats(torch, step, steps)
    gbps = bytes_step / (ms * 1e-3) / 1e9
    res = step_stats(ms, per)
    res.update({"us_per_layer": round(ms * 1e3 / wl.layers, 2),
                "tokens_per_s": round(wl.batch / (ms * 1e-3), 1), "gbps": round(gbps, 1),
                "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
                "live_rows": f"beacons {int(nb.min())}..{int(nb.max())} (mean {nb.mean():.0f}), raw "
                             f"{int(rw.min())}..{int(rw.max())} (mean {rw.mean():.0f}) + new token"})
    if page_rows:
        res["page_rows"] = page_rows
        del paged, tables
    log(f"{'paged' if page_rows else 'ragged'} step: {res}")
    del ws, step
    release(torch)
    return res


def chunk_step(lda, synth, torch, dev, wl, layers, steps, num_tokens, page_rows=0, even=False):
    """The ragged serving step of ragged_step with a chunk of num_tokens
    query tokens per sequence (e.g. drafted tokens checked in one pass):
    every layer attends each token over the live rows and the chunk's tokens
    up to it, and stores the tokens (slimkv_decode_attn_chunk).  page_rows >
    0: the cache lies in pages of that many rows at seeded, shuffled page
    ids (slimkv_decode_attn_chunk_paged).  Bytes: the live rows, the tokens'
    keys and values read and written, the queries, the bases, out and lse.
    even: every sequence at the drawn lengths' means instead (even_lengths)."""
    elem = wl.elem_bytes
    Q = num_tokens
    first = synth.make_step(wl, layers[0], device=dev, beacons=(0.5, 1.0), raw=(0.5, 1.0))
    if even:
        first = even_lengths(synth, wl, layers[0], dev, first)
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
        raws = [(x.K_raw.clone(), x.V_raw.clone()) for x in layers]  # the call stores tokens

        def step():
            for p, x, c, (kr, vr) in zip(probs, layers, chunks, raws):
                lda.slimkv_decode_attn_chunk(p, Q, c.q, x.q_pos, x.U_K, x.U_V, x.C_K, x.C_V,
                                             kr, vr, c.num_beacons, c.raw_len, c.k_new,
                                             c.v_new, out, lse, ws)

    ms, per = replay_stats(torch, step, steps)
    gbps = bytes_step / (ms * 1e-3) / 1e9
    res = {"tokens_per_chunk": Q}
    res.update(step_stats(ms, per))
    res.update({"us_per_layer": round(ms * 1e3 / wl.layers, 2),
                "query_tokens_per_s": round(wl.batch * Q / (ms * 1e-3), 1),
                "gbps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
                "live_rows": f"beacons {int(nb.min())}..{int(nb.max())} (mean {nb.mean():.0f}), raw "
                             f"{int(rw.min())}..{int(rw.max())} (mean {rw.mean():.0f}) + {Q} tokens"})
    if page_rows:
        res["page_rows"] = page_rows
        del paged, tables
    log(f"{'paged ' if page_rows else ''}chunk step: {res}")
    del ws, chunks, step
    release(torch)
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

    ms, per = replay_stats(torch, step, steps)
    total = sum(layer_call_bytes(wl, layer, elem)[1] for layer in range(wl.layers))
    gbps = total / (ms * 1e-3) / 1e9
    res = step_stats(ms, per)
    res.update({"us_per_layer": round(ms * 1e3 / wl.layers, 2),
                "tokens_per_s": round(wl.batch / (ms * 1e-3), 1), "gbps": round(gbps, 1),
                "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)})
    log(f"alibi step: {res}")
    del ws
    release(torch)
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

    ms, per = replay_stats(torch, step, steps)
    total = sum(layer_call_bytes(wl, layer, elem)[1] for layer in range(wl.layers))
    gbps = total / (ms * 1e-3) / 1e9
    res = step_stats(ms, per)
    res.update({"us_per_layer": round(ms * 1e3 / wl.layers, 2),
                "tokens_per_s": round(wl.batch / (ms * 1e-3), 1), "gbps": round(gbps, 1),
                "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)})
    log(f"{name} step: {res}")
    del layers, ws
    release(torch)
    return res


# ---------------------------------------------------------------------------
# The CPU baseline (the fp64 oracle on the host's cores) and the parity of
# the timed outputs.

BF16_MAX_ABS, BF16_REL_L2, FP32_REL_L2 = 1e-2, 5e-3, 1e-5


def cpu_baseline(wl, layers, budget_s, synth, last_out, last_lse):
    """The fp64 oracle on this host's cores over whole layers (the same
    inputs the GPU ran, copied to host memory once), in passes over the
    step's layers until the time budget is spent, starting with the last
    layer; the step time is the time per multiply-add times the step's
    multiply-add count (each layer's count depends on its rank).  The first
    call's result -- the last layer -- is compared with the out and lse the
    GPU's timed replays left behind: returns (baseline, parity)."""
    import numpy as np

    import oracle

    threads = oracle.max_threads()

    def macs(layer):
        r = wl.ranks[layer]
        per_head = wl.num_beacons * 2 * r + 2 * wl.raw_window * wl.head_dim + 2 * wl.head_dim * r
        return wl.batch * wl.num_q_heads * per_head

    st = synth.to_numpy_storage
    host = {}
    done, spent, calls = 0, 0.0, 0
    parity = None
    order = [wl.layers - 1] + list(range(wl.layers - 1))
    while spent < budget_s and calls < 64 * wl.layers:
        layer = order[calls % wl.layers]
        if layer not in host:
            x = layers[layer]
            host[layer] = [st(t) for t in (x.q, x.q_pos, x.U_K, x.U_V, x.C_K, x.C_V, x.K_raw,
                                           x.V_raw)]
        t0 = time.perf_counter()
        ref, ref_lse = oracle.decode(*host[layer], num_kv_heads=wl.num_kv_heads, scale=wl.scale,
                                     rope_theta=wl.rope_theta, threads=threads)
        spent += time.perf_counter() - t0
        if parity is None:
            diff = last_out - ref
            rel = float(np.linalg.norm(diff) / np.linalg.norm(ref))
            max_abs = float(np.abs(diff).max())
            per_head = np.linalg.norm(diff, axis=-1) / np.linalg.norm(ref, axis=-1)
            lse_err = float(np.abs(last_lse - ref_lse).max())
            bf16 = wl.dtype == "bf16"
            ok = (max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2) if bf16 else rel <= FP32_REL_L2
            parity = {"checked": f"layer {layer} (the step's last), all {wl.batch} x "
                                 f"{wl.num_q_heads} heads, GPU out/lse from the timed replays vs "
                                 "the fp64 oracle",
                      "rel_l2": float(f"{rel:.3e}"), "max_abs": float(f"{max_abs:.3e}"),
                      "worst_head_rel_l2": float(f"{float(per_head.max()):.3e}"),
                      "lse_max_abs": float(f"{lse_err:.3e}"),
                      "bar": ("max-abs <= 1e-2 and rel-L2 <= 5e-3" if bf16 else "rel-L2 <= 1e-5"),
                      "pass": bool(ok)}
            log(f"parity of the timed outputs: {parity}")
        done += macs(layer)
        calls += 1
    log(f"cpu oracle: {calls} layer calls in {spent:.1f}s")
    total = sum(macs(layer) for layer in range(wl.layers))
    step_s = spent * total / done
    passes = f"{calls / wl.layers:.2f} passes over the {wl.layers} layers"
    base = {"value": round(wl.batch / step_s, 3), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"{calls} layer calls ({passes}; all {wl.batch * wl.num_kv_heads} units "
                       f"each) timed in {spent:.1f}s with fp64 C+OpenMP; step time {step_s:.2f}s "
                       f"= time per multiply-add x the step's multiply-add count")}
    return base, parity


# ---------------------------------------------------------------------------
# Markdown report of bench results.

def _load_result(path):
    """(bench JSON line, source note) from a file: a driver record whose
    'parsed' holds the line (with the full line in the run's stdout), or a
    file whose last JSON line is the bench line."""
    text = pathlib.Path(path).read_text()
    try:
        rec = json.loads(text)
    except json.JSONDecodeError:
        rec = None
    if isinstance(rec, dict) and "run" in rec:
        line = None
        for ln in reversed(rec["run"].get("stdout_tail", "").splitlines()):
            if ln.startswith("{") and '"metric"' in ln:
                line = json.loads(ln)
                break
        line = line or rec.get("parsed", {})
        note = (f"{path}: driver run of `{rec.get('cmd', '')}` on {rec.get('where', '?')}, "
                f"commit {str(rec.get('head', '?'))[:12]}, {rec.get('driver_run_s', '?')} s")
        return line, note
    if isinstance(rec, dict) and "metric" in rec:
        return rec, str(path)
    for ln in reversed(text.splitlines()):
        if ln.startswith("{") and '"metric"' in ln:
            return json.loads(ln), str(path)
    raise SystemExit(f"{path}: no bench JSON line found")


def report(paths):
    out = ["# Benchmark report", "",
           "Generated by `python bench.py --report " + " ".join(paths) + "` from the files below; "
           "every figure is copied or derived from them. Peak HBM bandwidth of MI355X: 8 TB/s.", ""]
    for path in paths:
        r, note = _load_result(path)
        rf = r.get("roofline") or {}
        out += [f"## {r.get('config', {}).get('workload', '?').split(':')[0]}", "", f"Source: {note}", ""]
        out += ["| measure | value |", "|---|---|"]
        out.append(f"| decode-attention tokens/s (whole step, {r.get('config', {}).get('launch', '')}) "
                   f"| **{r.get('value')}** |")
        med = r.get("median_ms_per_step")
        pc = (f" (median {med}, p10 {r.get('p10_ms_per_step')}, p90 {r.get('p90_ms_per_step')})"
              if med is not None else "")
        out.append(f"| ms per step, mean over {r.get('steps')} steps | {r.get('ms_per_step')}{pc} |")
        out.append(f"| HBM GB/s over the step (algorithmic bytes) | {r.get('hbm_gbps')} "
                   f"({100 * r.get('hbm_frac_of_peak', 0):.1f}% of peak) |")
        if rf:
            out.append(f"| attention kernel, per launch (events) | {rf.get('launch_us')} us, "
                       f"{rf.get('achieved')} GB/s, **{100 * rf.get('frac', 0):.1f}% of peak** |")
            rp = rf.get("rocprof")
            if rp:
                out.append(f"| same, rocprofv3 kernel trace (`{rp.get('summary')}`) | "
                           f"{rp.get('launch_us')} us, {100 * rp.get('frac', 0):.1f}% of peak |")
            else:
                out.append("| same, rocprofv3 kernel trace | no committed trace for these kernel "
                           "sources |")
            tr = rf.get("traffic")
            ratio = tr / rf.get("bytes_per_launch", 1) if tr else 0.0
            out.append("| HBM traffic per launch (PMC) | " +
                       (f"{tr / 1e6:.1f} MB ({ratio:.3f} x algorithmic) |" if tr
                        else "not measured on these kernel sources |"))
            ce = rf.get("read_ceiling")
            if ce:
                out.append(f"| streaming-read ceiling, same bytes, one launch | {ce.get('us')} us, "
                           f"{ce.get('gbps')} GB/s ({100 * ce.get('frac_of_peak', 0):.1f}% of peak); "
                           f"attention kernel at {100 * rf.get('achieved', 0) / ce.get('gbps', 1):.1f}% "
                           f"of it |")
        other = [k for k in r if k.startswith("step_")]
        for k in other:
            o = r[k]
            out.append(f"| same step, {o.get('launch')} | {o.get('ms_per_step')} ms, "
                       f"{o.get('tokens_per_s')} tokens/s |")
        cb = r.get("cpu_baseline")
        if cb:
            out.append(f"| CPU oracle (fp64, {cb.get('cores')} host threads) | {cb.get('value')} "
                       f"{cb.get('unit')}: {cb.get('sample')} |")
        par = r.get("parity")
        if par:
            out.append(f"| parity of the timed outputs ({par.get('checked')}) | rel-L2 "
                       f"{par.get('rel_l2')}, max-abs {par.get('max_abs')}, lse {par.get('lse_max_abs')}; "
                       f"bar {par.get('bar')}: **{'pass' if par.get('pass') else 'FAIL'}** |")
        out.append("")
        cmp_ = r.get("comparison") or {}
        one = {k: v for k, v in cmp_.items() if k in ("full_kv", "c2") or k.startswith("c5_")}
        if one:
            out += ["### One layer at 128K (B 16), inputs rotated over copies > 1 GB", "",
                    "| path | us (median, p10-p90) | GB/s | % of peak | speedup |", "|---|---|---|---|---|"]
            for k, v in one.items():
                sp = []
                if "speedup_vs_full_kv" in v:
                    sp.append(f"{v['speedup_vs_full_kv']}x vs full KV")
                if "speedup_vs_reconstruct" in v:
                    sp.append(f"{v['speedup_vs_reconstruct']}x vs reconstruct")
                if "speedup_vs_reconstruct_rope" in v:
                    sp.append(f"{v['speedup_vs_reconstruct_rope']}x vs reconstruct with beacon RoPE")
                out.append(f"| {k} | {v.get('us')} ({v.get('median_us')}, {v.get('p10_us')}-"
                           f"{v.get('p90_us')}) | {v.get('gbps')} | "
                           f"{100 * v.get('frac_of_peak', 0):.1f} | {'; '.join(sp)} |")
                for sub in ("reconstruct", "reconstruct_rope"):
                    if sub in v:
                        w = v[sub]
                        out.append(f"| {k} {sub.replace('_', ' ')} | {w.get('us')} ({w.get('median_us')}, "
                                   f"{w.get('p10_us')}-{w.get('p90_us')}) | {w.get('gbps')} | "
                                   f"{100 * w.get('frac_of_peak', 0):.1f} | baseline |")
            out.append("")
        steps = {k: v for k, v in cmp_.items() if k not in one}
        if steps:
            out += ["### Other whole steps (graph replay)", "",
                    "| step | ms (median) | us per layer | rate | GB/s | % of peak |",
                    "|---|---|---|---|---|---|"]
            for k, v in steps.items():
                rate = v.get("tokens_per_s") or v.get("query_tokens_per_s")
                out.append(f"| {k} | {v.get('ms_per_step')} ({v.get('median_ms')}) | "
                           f"{v.get('us_per_layer')} | {rate} | {v.get('gbps')} | "
                           f"{100 * v.get('frac_of_peak', 0):.1f} |")
            out.append("")
    # the lines themselves, so that the report can be checked (and remade
    # with --report from a file holding one of them)
    out += ["## Source lines", ""]
    for path in paths:
        r, note = _load_result(path)
        out += [f"{note}:", "", "```json", json.dumps(r), "```", ""]
    return "\n".join(out) + "\n"


# ---------------------------------------------------------------------------
# rocprofv3 kernel-trace summary.

def kernel_name(full):
    """A trace's kernel name without its parameter list and return type."""
    anon = "(anonymous namespace)"
    name = full.replace(anon, "\x00").split("(")[0].replace("\x00", anon)
    return name[5:] if name.startswith("void ") else name


def headline_dispatches(items, wl, steps, other_warm=2):
    """The attention dispatches of the headline's timed steps in a bench run
    with --no-compare --no-cpu-baseline (in launch order): after them the
    bench times the other launch form, ``other_warm`` warm-up steps (its
    JSON line's warmup_steps_run.other) and ``steps`` steps, which are
    skipped.  Within a step the dispatches follow the layers in order, so
    dispatch i of a step is layer i and its bytes are known."""
    n, other = steps * wl.layers, (steps + other_warm) * wl.layers
    if len(items) < n + other:
        raise SystemExit(f"{len(items)} attention dispatches, fewer than the {n} timed and "
                         f"{other} after them that a bench run with --steps {steps} makes")
    return items[len(items) - other - n:len(items) - other]


def profile_summary(directory, wl, steps, other_warm=2):
    """The attention kernel's dispatches in a rocprofv3 kernel trace (CSV)
    of the headline's timed steps (headline_dispatches).  Durations are End -
    Start of each dispatch, in us; every other kernel is listed with its
    totals."""
    import csv

    import numpy as np
    files = sorted(glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no *kernel_trace.csv under {directory}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                rows.append((int(row["Start_Timestamp"]), int(row["End_Timestamp"]),
                             kernel_name(row["Kernel_Name"])))
    rows.sort()
    att = [r for r in rows if "attention_kernel" in r[2]]
    last = headline_dispatches(att, wl, steps, other_warm)
    n = len(last)
    dur = np.array([(e - s) / 1e3 for s, e, _ in last]).reshape(steps, wl.layers)
    elem = wl.elem_bytes
    per_layer = []
    for layer in range(wl.layers):
        b = layer_call_bytes(wl, layer, elem)[1]
        us = float(dur[:, layer].mean())
        per_layer.append({"layer": layer, "rank": wl.ranks[layer], "kernel": last[layer][2],
                          "avg_us": round(us, 2), "bytes": b,
                          "gbps": round(b / (us * 1e-6) / 1e9, 1)})
    step_sum = dur.sum(axis=1)
    span = (last[-1][1] - last[0][0]) / 1e3 / steps
    launch_us = float(dur.mean())
    mean_bytes = sum(layer_call_bytes(wl, layer, elem)[1] for layer in range(wl.layers)) / wl.layers
    gbps = mean_bytes / (launch_us * 1e-6) / 1e9
    by_rank = {}
    for p in per_layer:
        by_rank.setdefault(p["rank"], []).append(p)
    ranks = {str(r): {"layers": len(ps), "kernel": ps[0]["kernel"],
                      "avg_us": round(float(np.mean([p["avg_us"] for p in ps])), 2),
                      "bytes": ps[0]["bytes"],
                      "gbps": round(ps[0]["bytes"] / (float(np.mean([p["avg_us"] for p in ps]))
                                                      * 1e-6) / 1e9, 1)}
             for r, ps in sorted(by_rank.items())}
    others = {}
    for s, e, name in rows:
        if "attention_kernel" not in name:
            o = others.setdefault(name[:80], [0, 0.0])
            o[0] += 1
            o[1] += (e - s) / 1e3
    return {"kind": "kernel_trace", "kernel": "attention_kernel", "workload": wl.name,
            "steps": steps, "dispatches": n,
            "launch_us": round(launch_us, 3), "gbps": round(gbps, 1),
            "frac": round(gbps / HBM_PEAK_GBPS, 4), "bytes_per_launch": int(mean_bytes),
            "kernel_sum_per_step_us": round(float(step_sum.mean()), 1),
            "traced_step_ms": round(span / 1e3, 4),
            "first_start_to_last_end_per_step_us": round(span, 1),
            "per_rank": ranks, "per_layer": per_layer,
            "other_kernels": {k: {"calls": v[0], "sum_us": round(v[1], 1)} for k, v in others.items()},
            "files": [os.path.relpath(f, directory) for f in files]}


def read_counters(directory):
    """Per dispatch of a rocprofv3 --pmc run (*counter_collection.csv under
    directory): (dispatch id, kernel name, {counter: value}), in dispatch
    order."""
    import csv
    files = sorted(glob.glob(os.path.join(directory, "**", "*counter_collection.csv"),
                             recursive=True))
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {directory}")
    by = {}
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                d = by.setdefault(int(row["Dispatch_Id"]), [kernel_name(row["Kernel_Name"]), {}])
                d[1][row["Counter_Name"]] = d[1].get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    return [(k, v[0], v[1]) for k, v in sorted(by.items())]


def calibration_scales(cal_fetch_dir, cal_write_dir):
    """Bytes per counter KiB: FETCH_SIZE of the library's plain read kernel
    over 1 GiB - 16 bytes and WRITE_SIZE of its write kernel over 1 GiB
    (bench.py --calibrate), medians over their dispatches; and the FETCH_SIZE
    of the torch copy of 1 GiB (a cross-check)."""
    import numpy as np
    cal_f = [(n, c["FETCH_SIZE"]) for _, n, c in read_counters(cal_fetch_dir) if "FETCH_SIZE" in c]
    cal_w = [(n, c["WRITE_SIZE"]) for _, n, c in read_counters(cal_write_dir) if "WRITE_SIZE" in c]

    def median_of(rows, key):
        vals = [v for name, v in rows if key in name]
        if not vals:
            raise SystemExit(f"no calibration dispatch named *{key}*")
        return float(np.median(vals))
    gib = 1 << 30
    copy_f = [v for name, v in cal_f if "stream_read" not in name and "flush" not in name]
    return ((gib - 16) / (median_of(cal_f, "stream_read_kernel") * 1024),
            gib / (median_of(cal_w, "flush_kernel") * 1024),
            float(np.median(copy_f)) if copy_f else None)


def instance_trace_summary(directory, kernel):
    """Every dispatch of ``kernel`` in a rocprofv3 kernel trace, per
    instance: calls, mean / min / max duration in us."""
    import csv

    import numpy as np
    files = sorted(glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no *kernel_trace.csv under {directory}")
    by = {}
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                name = kernel_name(row["Kernel_Name"])
                if kernel in name:
                    by.setdefault(name, []).append(
                        (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3)
    if not by:
        raise SystemExit(f"no dispatch of {kernel} under {directory}")
    inst = {k: {"calls": len(v), "avg_us": round(float(np.mean(v)), 2),
                "min_us": round(float(np.min(v)), 2), "max_us": round(float(np.max(v)), 2)}
            for k, v in sorted(by.items())}
    allv = [x for v in by.values() for x in v]
    return {"kind": "instance_trace", "kernel": kernel, "workload": "",
            "dispatches": len(allv), "launch_us": round(float(np.mean(allv)), 2), "instances": inst,
            "files": [os.path.relpath(f, directory) for f in files]}


def instance_traffic_summary(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, kernel):
    """FETCH_SIZE and WRITE_SIZE of every dispatch of ``kernel``, per
    instance, scaled to bytes by calibration_scales."""
    import numpy as np
    rs, ws_, copy_kib = calibration_scales(cal_fetch_dir, cal_write_dir)
    by = {}
    for counter, directory in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        for _, name, c in read_counters(directory):
            if kernel in name and counter in c:
                by.setdefault(name, {}).setdefault(counter, []).append(c[counter])
    if not by:
        raise SystemExit(f"no counters for {kernel}")
    inst = {}
    rd_all, wr_all = [], []
    for name, c in sorted(by.items()):
        f, w = c.get("FETCH_SIZE", [0.0]), c.get("WRITE_SIZE", [0.0])
        rd_all += [x * 1024 * rs for x in f]
        wr_all += [x * 1024 * ws_ for x in w]
        inst[name] = {"dispatches": len(f), "fetch_kib": round(float(np.mean(f)), 1),
                      "write_kib": round(float(np.mean(w)), 1),
                      "read_mb": round(float(np.mean(f)) * 1024 * rs / 1e6, 2),
                      "write_mb": round(float(np.mean(w)) * 1024 * ws_ / 1e6, 2)}
    return {"kind": "instance_traffic", "kernel": kernel, "workload": "", "fetch_scale": round(rs, 4),
            "write_scale": round(ws_, 4),
            "copy_fetch_kib_per_gib": round(copy_kib, 1) if copy_kib else None,
            "read_bytes_per_launch": int(np.mean(rd_all)), "write_bytes_per_launch": int(np.mean(wr_all)),
            "traffic_bytes_per_launch": int(np.mean(rd_all) + np.mean(wr_all)), "instances": inst}


def traffic_summary(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, wl, steps, other_warm=(2, 2)):
    """HBM bytes of the attention kernel from FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch, one counter per run), each scaled by what the same
    counter reads for the calibration kernels of known size (bench.py
    --calibrate: the library's plain read kernel for reads, its flush kernel
    for writes; the torch copy is a cross-check).  The dispatches are the
    headline's timed steps (headline_dispatches), so each one's layer and
    algorithmic bytes are known."""
    import numpy as np

    def one(directory, counter):
        return [(name, c[counter]) for _, name, c in read_counters(directory) if counter in c]

    read_scale, write_scale, copy_kib = calibration_scales(cal_fetch_dir, cal_write_dir)
    fetch = headline_dispatches([r for r in one(fetch_dir, "FETCH_SIZE") if "attention_kernel" in r[0]],
                                wl, steps, other_warm[0])
    write = headline_dispatches([r for r in one(write_dir, "WRITE_SIZE") if "attention_kernel" in r[0]],
                                wl, steps, other_warm[1])
    elem = wl.elem_bytes
    per_rank = {}
    rd_all, wr_all, alg_all = [], [], []
    for i, ((name, f), (_, w)) in enumerate(zip(fetch, write)):
        layer = i % wl.layers
        alg = layer_call_bytes(wl, layer, elem)[1]
        rd, wr = f * 1024 * read_scale, w * 1024 * write_scale
        rd_all.append(rd)
        wr_all.append(wr)
        alg_all.append(alg)
        e = per_rank.setdefault(str(wl.ranks[layer]), {"kernel": name, "dispatches": 0, "fetch_kib": [],
                                                        "write_kib": [], "alg": alg})
        e["dispatches"] += 1
        e["fetch_kib"].append(f)
        e["write_kib"].append(w)
    ranks = {}
    for r, e in sorted(per_rank.items(), key=lambda x: int(x[0])):
        fk, wk = float(np.mean(e["fetch_kib"])), float(np.mean(e["write_kib"]))
        ranks[r] = {"kernel": e["kernel"], "dispatches": e["dispatches"], "fetch_kib": round(fk, 1),
                    "write_kib": round(wk, 1), "read_mb": round(fk * 1024 * read_scale / 1e6, 2),
                    "write_mb": round(wk * 1024 * write_scale / 1e6, 2),
                    "algorithmic_mb": round(e["alg"] / 1e6, 2),
                    "read_over_algorithmic": round(fk * 1024 * read_scale / e["alg"], 4)}
    traffic = float(np.mean(rd_all) + np.mean(wr_all))
    alg = float(np.mean(alg_all))
    return {"kind": "pmc_traffic", "kernel": "attention_kernel", "workload": wl.name, "steps": steps,
            "dispatches": len(fetch), "fetch_scale": round(read_scale, 4),
            "write_scale": round(write_scale, 4),
            "copy_fetch_kib_per_gib": round(copy_kib, 1) if copy_kib else None,
            "traffic_bytes_per_launch": int(traffic), "read_bytes_per_launch": int(np.mean(rd_all)),
            "write_bytes_per_launch": int(np.mean(wr_all)), "algorithmic_bytes_per_launch": int(alg),
            "traffic_over_algorithmic": round(traffic / alg, 4), "per_rank": ranks}


def other_warm(files, i):
    """Warm-up steps of the other launch form in the profiled run whose
    JSON line is files[i] (2, the count before the warm-up had a time floor,
    if not given)."""
    if i >= len(files):
        return 2
    with open(files[i]) as fh:
        line = json.loads(fh.read().strip().splitlines()[-1])
    return int(line.get("warmup_steps_run", {}).get("other", 2))


def write_record(name, summ, args):
    """profiles/NAME.json (the summary, stamped with the kernel sources'
    sha256) and profiles/NAME.md (the same as a table, with the commands)."""
    rec = dict(summ)
    rec["source_sha256"] = source_sha256()
    rec["commands"] = args.command or []
    untraced = None
    if args.untraced:
        with open(args.untraced) as fh:
            untraced = json.loads(fh.read().strip().splitlines()[-1])
        rec["untraced"] = {k: untraced.get(k) for k in ("ms_per_step", "median_ms_per_step",
                                                         "value", "unit")}
        rec["untraced"]["launch_us"] = untraced.get("roofline", {}).get("launch_us")
    rec["summary"] = f"profiles/{name}.md"
    if not rec["workload"]:
        rec["workload"] = args.label or args.record
    out = pathlib.Path(ROOT) / "profiles"
    (out / f"{name}.json").write_text(json.dumps(rec, indent=1) + "\n")
    kind = rec["kind"]
    lines = [f"# {rec['kernel']} on {rec['workload']}: "
             + ("kernel trace" if kind.endswith("trace") else "HBM traffic (PMC)"), ""]
    lines += ["Commands (repository root, MI355X):", ""]
    lines += [f"    {c}" for c in rec["commands"]] + [""]
    lines += [f"Kernel source sha256 (latent_decode_attention_amd/csrc): `{rec['source_sha256']}`", ""]
    if kind == "instance_trace":
        lines += [f"Every dispatch of {rec['kernel']} in the run ({rec['dispatches']}), per instance.",
                  "", "| kernel instance | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
        for k, e in rec["instances"].items():
            lines.append(f"| {k} | {e['calls']} | {e['avg_us']} | {e['min_us']} | {e['max_us']} |")
        lines += ["", f"Average over all dispatches: **{rec['launch_us']} us**."]
        if args.algorithmic_bytes:
            gbps = args.algorithmic_bytes / (rec["launch_us"] * 1e-6) / 1e9
            rec["algorithmic_bytes_per_launch"] = int(args.algorithmic_bytes)
            rec["gbps"] = round(gbps, 1)
            rec["frac"] = round(gbps / HBM_PEAK_GBPS, 4)
            (out / f"{name}.json").write_text(json.dumps(rec, indent=1) + "\n")
            lines += [f"Algorithmic bytes per dispatch (given): {args.algorithmic_bytes / 1e6:.1f} MB -> "
                      f"{gbps:.1f} GB/s = **{100 * gbps / HBM_PEAK_GBPS:.1f}% of 8 TB/s**."]
        if untraced:
            lines += ["", "The same command without the profiler on the same box: "
                      + json.dumps({k: v for k, v in untraced.items()
                                    if k in ("ms_per_step", "median_ms", "us_per_layer", "us", "gbps",
                                             "frac_of_peak", "live_rows", "tokens_per_chunk",
                                             "reconstruct", "reconstruct_rope")})]
    elif kind == "instance_traffic":
        lines += [f"Scale from counter units to bytes: reads x{rec['fetch_scale']}, writes "
                  f"x{rec['write_scale']} (bench.py --calibrate).", "",
                  "| kernel instance | dispatches | FETCH KiB | WRITE KiB | read MB | write MB |",
                  "|---|---|---|---|---|---|"]
        for k, e in rec["instances"].items():
            lines.append(f"| {k} | {e['dispatches']} | {e['fetch_kib']} | {e['write_kib']} | "
                         f"{e['read_mb']} | {e['write_mb']} |")
        lines += ["", f"Per dispatch over the run: read {rec['read_bytes_per_launch'] / 1e6:.1f} MB + "
                  f"write {rec['write_bytes_per_launch'] / 1e6:.2f} MB."]
        live = args.algorithmic_bytes or (untraced["gbps"] * untraced["us_per_layer"] * 1e3
                                          if untraced and untraced.get("gbps")
                                          and untraced.get("us_per_layer") else 0.0)
        if live:
            lines += [f"Algorithmic bytes per dispatch ("
                      f"{'given' if args.algorithmic_bytes else 'the live bytes per layer of the untraced run'}): "
                      f"{live / 1e6:.1f} MB; measured / algorithmic = "
                      f"{rec['traffic_bytes_per_launch'] / live:.3f}."]
            rec["algorithmic_bytes_per_launch"] = int(live)
            (out / f"{name}.json").write_text(json.dumps(rec, indent=1) + "\n")
    elif kind == "kernel_trace":
        lines += [f"{rec['dispatches']} dispatches: the headline's {rec['steps']} timed steps x "
                  f"{rec['dispatches'] // rec['steps']} layers.", "",
                  "| ranks | kernel instance | layers | avg us | algorithmic MB/launch | GB/s |",
                  "|---|---|---|---|---|---|"]
        for r, e in rec["per_rank"].items():
            lines.append(f"| {r} | {e['kernel']} | {e['layers']} | {e['avg_us']} | "
                         f"{e['bytes'] / 1e6:.1f} | {e['gbps']} |")
        lines += ["", f"Average over the step's layers: **{rec['launch_us']} us per launch**, "
                  f"{rec['bytes_per_launch'] / 1e6:.1f} MB algorithmic -> {rec['gbps']} GB/s = "
                  f"**{100 * rec['frac']:.2f}% of 8 TB/s**.",
                  f"Per step: kernel durations sum to {rec['kernel_sum_per_step_us']} us; first "
                  f"start to last end {rec['first_start_to_last_end_per_step_us']} us."]
        if untraced:
            lines += ["", f"The same command without the profiler on the same box: "
                      f"{untraced.get('ms_per_step')} ms per step (events over the timed region, "
                      f"gaps between launches included), {rec['untraced']['launch_us']} us per "
                      f"launch. The traced kernel sum per step is "
                      f"{rec['kernel_sum_per_step_us'] / 1e3 / untraced.get('ms_per_step'):.3f} "
                      f"of that step."]
    else:
        lines += [f"Scale from counter units to bytes: reads x{rec['fetch_scale']} (the library's "
                  f"plain read kernel over 1 GiB), writes x{rec['write_scale']} (its write kernel over "
                  f"1 GiB); a torch copy of 1 GiB reads {rec['copy_fetch_kib_per_gib']} KiB of "
                  f"FETCH_SIZE.", "",
                  "| ranks | kernel instance | dispatches | FETCH KiB | WRITE KiB | read MB | write MB | "
                  "algorithmic MB | read / algorithmic |", "|---|---|---|---|---|---|---|---|---|"]
        for r, e in rec["per_rank"].items():
            lines.append(f"| {r} | {e['kernel']} | {e['dispatches']} | {e['fetch_kib']} | "
                         f"{e['write_kib']} | {e['read_mb']} | {e['write_mb']} | "
                         f"{e['algorithmic_mb']} | {e['read_over_algorithmic']} |")
        lines += ["", f"Per launch over the step's layers: read {rec['read_bytes_per_launch'] / 1e6:.1f} "
                  f"MB + write {rec['write_bytes_per_launch'] / 1e6:.2f} MB = "
                  f"**{rec['traffic_bytes_per_launch'] / 1e6:.1f} MB**, against "
                  f"{rec['algorithmic_bytes_per_launch'] / 1e6:.1f} MB algorithmic "
                  f"({rec['traffic_over_algorithmic']}x)."]
    (out / f"{name}.md").write_text("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
