"""Write the oracle regression fixtures in this folder.

The pages print no worked example of the attention itself (their figures
are latencies, memory footprints and benchmark scores), so no fixture here
holds a value from the pages.  These fixtures hold the fp64 oracle's
outputs on tiny seeded inputs (synth's generators, parameters stored with
each case), one per oracle entry point, so that any later change to the
oracle's arithmetic shows up as a failing test and is made deliberately:
regenerate with ``python tests/golden/make_golden.py`` and name, in the
commit, the passage that justifies the change.  Only synth (inputs) and the
oracle are used.
"""

import dataclasses
import json
import pathlib
import sys

import numpy as np

ROOT = pathlib.Path(__file__).resolve().parents[2]
sys.path.insert(0, str(ROOT))

import oracle  # noqa: E402
import synth  # noqa: E402

HERE = pathlib.Path(__file__).resolve().parent


def workload(dtype, B, Hkv, G, nb, w, r, context, index):
    return dataclasses.replace(
        synth.get_workload("c2"), name="golden", index=index, batch=B, num_q_heads=Hkv * G,
        num_kv_heads=Hkv, num_beacons=nb, raw_window=w, ranks=(r,), dtype=dtype, sigma=1.0,
        context=context)


CASES = {
    # name: (entry point, workload parameters, extra)
    "decode_bf16": ("decode", dict(dtype="bf16", B=2, Hkv=1, G=2, nb=7, w=5, r=32,
                                   context=4096, index=400), {}),
    "decode_ragged_fp32": ("decode_ragged", dict(dtype="fp32", B=3, Hkv=1, G=2, nb=6, w=4, r=16,
                                                 context=4096, index=401),
                           dict(fixed={0: (6, 4), 1: (2, 0), 2: (0, 3)})),
    "decode_chunk_bf16": ("decode_chunk", dict(dtype="bf16", B=2, Hkv=1, G=2, nb=5, w=6, r=32,
                                               context=4096, index=402),
                          dict(tokens=2, fixed={0: (5, 3), 1: (1, 6)})),
    "decode_alibi_bf16": ("decode_alibi", dict(dtype="bf16", B=2, Hkv=1, G=2, nb=6, w=4, r=16,
                                               context=200, index=403), dict(ratio=16)),
    "decode_chunk_fp32": ("decode_chunk", dict(dtype="fp32", B=2, Hkv=1, G=2, nb=4, w=5, r=16,
                                               context=4096, index=404),
                          dict(tokens=3, fixed={0: (4, 2), 1: (0, 5)})),
    "decode_chunk_alibi_bf16": ("decode_chunk_alibi", dict(dtype="bf16", B=2, Hkv=1, G=2, nb=6,
                                                           w=5, r=16, context=300, index=405),
                                dict(tokens=2, ratio=16, fixed={0: (6, 3), 1: (2, 5)})),
}


def run_case(name):
    """The oracle's outputs for case ``name`` (inputs regenerated from its
    parameters): a dict of float64 lists."""
    entry, params, extra = CASES[name]
    wl = workload(**params)
    inp = synth.make_layer(wl)
    st = synth.to_numpy_storage
    nb, w = inp.num_beacons, inp.raw_window
    common = (st(inp.U_K), st(inp.U_V), st(inp.C_K) if nb else None, st(inp.C_V) if nb else None,
              st(inp.K_raw) if w else None, st(inp.V_raw) if w else None)
    kw = dict(num_kv_heads=wl.num_kv_heads, scale=wl.scale)
    if entry == "decode":
        out, lse = oracle.decode(st(inp.q), st(inp.q_pos), *common, rope_theta=wl.rope_theta, **kw)
        res = dict(out=out, lse=lse)
    elif entry == "decode_ragged":
        step = synth.make_step(wl, inp, fixed=extra["fixed"])
        out, lse, k_app = oracle.decode_ragged(
            st(inp.q), st(inp.q_pos), *common, rope_theta=wl.rope_theta,
            num_beacons=st(step.num_beacons), raw_len=st(step.raw_len), k_new=st(step.k_new),
            v_new=st(step.v_new), **kw)
        res = dict(out=out, lse=lse, k_app=k_app)
    elif entry == "decode_chunk":
        ch = synth.make_chunk(wl, inp, extra["tokens"], fixed=extra["fixed"])
        out, lse, k_app = oracle.decode_chunk(
            st(ch.q), st(inp.q_pos), *common, rope_theta=wl.rope_theta,
            num_beacons=st(ch.num_beacons), raw_len=st(ch.raw_len), k_new=st(ch.k_new),
            v_new=st(ch.v_new), **kw)
        res = dict(out=out, lse=lse, k_app=k_app)
    elif entry == "decode_chunk_alibi":
        ch = synth.make_chunk(wl, inp, extra["tokens"], fixed=extra["fixed"])
        first, stride = synth.beacon_grid(extra["ratio"])
        slopes = synth.alibi_slopes(wl.num_q_heads).astype(np.float32).astype(np.float64)
        out, lse, k_app = oracle.decode_chunk_alibi(
            st(ch.q), st(inp.q_pos), *common,
            beacon_pos=(first + stride * np.arange(nb)).astype(np.int32), slopes=slopes,
            num_beacons=st(ch.num_beacons), raw_len=st(ch.raw_len), k_new=st(ch.k_new),
            v_new=st(ch.v_new), **kw)
        res = dict(out=out, lse=lse, k_app=k_app)
    else:
        first, stride = synth.beacon_grid(extra["ratio"])
        slopes = synth.alibi_slopes(wl.num_q_heads).astype(np.float32).astype(np.float64)
        out, lse = oracle.decode_alibi(
            st(inp.q), st(inp.q_pos), *common,
            beacon_pos=(first + stride * np.arange(nb)).astype(np.int32), slopes=slopes, **kw)
        res = dict(out=out, lse=lse)
    return {k: np.asarray(v, dtype=np.float64) for k, v in res.items()}


def main():
    for name, (entry, params, extra) in CASES.items():
        res = run_case(name)
        doc = {"case": name, "entry": entry, "params": params,
               "extra": {k: ({str(b): list(v) for b, v in x.items()} if k == "fixed" else x)
                         for k, x in extra.items()},
               "shapes": {k: list(v.shape) for k, v in res.items()},
               "values": {k: [float(x) for x in v.ravel()] for k, v in res.items()}}
        (HERE / f"{name}.json").write_text(json.dumps(doc, indent=None) + "\n")
        print("wrote", name)


if __name__ == "__main__":
    main()
