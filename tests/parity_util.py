"""Helpers for the GPU parity tests: run the HIP library and the fp64 oracle
on the same seeded inputs and compare.

Tolerances (floating point; nothing here decides an integer):
  * bf16 caches, fp32 accumulation: max-abs <= 1e-2 and relative L2 <= 5e-3
    over the call's whole output (or over the sampled units);
  * fp32: relative L2 <= 1e-5;
  * lse: |error| <= LSE_TOL[dtype] * max(1, |lse|).  The kernels score with
    a two-term bf16 split of the fp32 query (about 2^-17 relative) against
    exact storage keys, accumulate in fp32 and take exp2 in fp32, so score
    errors stay near 1e-6 * |score| and the log-sum-exp inherits that.
  * the reconstruction path rounds each rebuilt beacon key element to bf16
    (relative 2^-9), which moves every beacon score by up to about
    2^-8 * |score|; its lse tolerance is RECON_LSE_TOL * max(1, |lse|).
"""

from __future__ import annotations

import dataclasses
import sys

import numpy as np
import torch

import latent_decode_attention_amd as lda
import oracle
import synth

TOL = {"fp32": dict(rel_l2=1e-5, max_abs=None), "bf16": dict(rel_l2=5e-3, max_abs=1e-2)}
LSE_TOL = {"fp32": 1e-5, "bf16": 1e-4}
RECON_LSE_TOL = {"fp32": 1e-5, "bf16": 1e-2}


def note(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run says where."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def run_gpu(inp: synth.LayerInputs, op: int = lda.SLIMKV_OP_LATENT, *, num_splits: int = 0,
            device="cuda", with_lse: bool = True, full_k=None, full_v=None, flags: int = 0,
            beacon_pos=None):
    """Run one entry point on ``inp`` (moved to the GPU if needed).  With
    op = RECONSTRUCT and beacon_pos ([N_b] int32), the variant that rotates
    the rebuilt beacon keys (slimkv_reconstruct_rope_attn)."""
    wl = inp.workload
    g = inp.to(device)
    if op == lda.SLIMKV_OP_FULL_KV:
        K, V = full_k.to(device), full_v.to(device)
        prob = lda.make_problem(batch=wl.batch, num_q_heads=wl.num_q_heads,
                                num_kv_heads=wl.num_kv_heads, num_beacons=0, rank_k=0, rank_v=0,
                                raw_window=int(K.shape[2]), scale=wl.scale,
                                rope_theta=wl.rope_theta, dtype=wl.dtype, num_splits=num_splits,
                                flags=flags)
    else:
        prob = lda.problem_from_tensors(g.q, g.U_K, g.C_K, g.K_raw, U_V=g.U_V,
                                        rope_theta=wl.rope_theta, num_kv_heads=wl.num_kv_heads,
                                        scale=wl.scale, num_splits=num_splits, flags=flags)
    out, lse = lda.alloc_outputs(prob, device)
    ws = lda.alloc_workspace(prob, op, device)
    if not with_lse:
        lse = None
    if op == lda.SLIMKV_OP_LATENT:
        lda.slimkv_decode_attn(prob, g.q, g.q_pos, g.U_K, g.U_V, g.C_K, g.C_V, g.K_raw, g.V_raw,
                               out, lse, ws)
    elif op == lda.SLIMKV_OP_RECONSTRUCT and beacon_pos is not None:
        lda.slimkv_reconstruct_rope_attn(prob, g.q, g.q_pos, g.U_K, g.U_V, g.C_K, g.C_V, g.K_raw,
                                         g.V_raw, beacon_pos.to(device), out, lse, ws)
    elif op == lda.SLIMKV_OP_RECONSTRUCT:
        lda.slimkv_reconstruct_attn(prob, g.q, g.q_pos, g.U_K, g.U_V, g.C_K, g.C_V, g.K_raw,
                                    g.V_raw, out, lse, ws)
    else:
        lda.full_kv_attn(prob, g.q, g.q_pos, K, V, out, lse, ws)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), (None if lse is None else lse.double().cpu().numpy())


def oracle_layer(inp: synth.LayerInputs, units=None, threads: int = 0, beacon_pos=None):
    """Oracle on the whole layer (inputs copied to the host), or on a list of
    (b, kv head) units; beacon_pos selects the rotated-beacon reconstruction."""
    wl = inp.workload
    st = synth.to_numpy_storage
    nb, w = inp.num_beacons, inp.raw_window
    return oracle.decode(st(inp.q), st(inp.q_pos), st(inp.U_K), st(inp.U_V),
                         st(inp.C_K) if nb else None, st(inp.C_V) if nb else None,
                         st(inp.K_raw) if w else None, st(inp.V_raw) if w else None,
                         num_kv_heads=wl.num_kv_heads, scale=wl.scale, rope_theta=wl.rope_theta,
                         units=units, threads=threads,
                         beacon_pos=None if beacon_pos is None else st(beacon_pos))


def oracle_units(inp: synth.LayerInputs, units, beacon_pos=None):
    """Oracle on sampled units, copying only each unit's slices to the host.
    Returns {(b, h): (out [G, d], lse [G])}."""
    wl = inp.workload
    res = {}
    for b, h in units:
        s = synth.unit_slices(inp, b, h)
        nb, w = s["C_K"].shape[2], s["K_raw"].shape[2]
        o, l = oracle.decode(s["q"], s["q_pos"], s["U_K"], s["U_V"], s["C_K"] if nb else None,
                             s["C_V"] if nb else None, s["K_raw"] if w else None,
                             s["V_raw"] if w else None, num_kv_heads=1, scale=wl.scale,
                             rope_theta=wl.rope_theta,
                             beacon_pos=None if beacon_pos is None
                             else synth.to_numpy_storage(beacon_pos))
        res[(b, h)] = (o[0], l[0])
    return res


def beacon_positions(num_beacons: int, context: int) -> torch.Tensor:
    """One beacon per s = context / num_beacons tokens, at the last position
    of its span: (j + 1) s - 1."""
    s = max(context // max(num_beacons, 1), 1)
    return ((torch.arange(num_beacons, dtype=torch.int64) + 1) * s - 1).to(torch.int32)


def oracle_full_kv_units(wl, q, q_pos, K, V, units):
    """Oracle for uncompressed attention on sampled units (raw-only problem)."""
    st = synth.to_numpy_storage
    G = wl.group
    res = {}
    for b, h in units:
        o, l = oracle.decode(st(q[b:b + 1, h * G:(h + 1) * G]), st(q_pos[b:b + 1]), None, None,
                             None, None, st(K[b:b + 1, h:h + 1]), st(V[b:b + 1, h:h + 1]),
                             num_kv_heads=1, scale=wl.scale, rope_theta=wl.rope_theta)
        res[(b, h)] = (o[0], l[0])
    return res


def errors(got: np.ndarray, ref: np.ndarray):
    diff = got - ref
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    return rel, float(np.max(np.abs(diff)))


def assert_parity(got, ref, dtype: str, what: str = "", lse=None, lse_ref=None, lse_tol=None):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rel, mx = errors(got, ref)
    tol = TOL[dtype]
    print(f"[parity] {what}: rel_l2={rel:.3e} max_abs={mx:.3e}", flush=True)
    assert rel <= tol["rel_l2"], f"{what}: rel-L2 {rel:.3e} > {tol['rel_l2']}"
    if tol["max_abs"] is not None:
        assert mx <= tol["max_abs"], f"{what}: max-abs {mx:.3e} > {tol['max_abs']}"
    if lse is not None:
        lerr = np.abs(lse - lse_ref) / np.maximum(1.0, np.abs(lse_ref))
        print(f"[parity] {what}: lse max scaled err={lerr.max():.3e}", flush=True)
        tol_l = LSE_TOL[dtype] if lse_tol is None else lse_tol
        assert lerr.max() <= tol_l, f"{what}: lse error {lerr.max():.3e} > {tol_l}"


def sample_units(wl, n: int, seed: int):
    rng = np.random.default_rng(seed)
    all_units = [(b, h) for b in range(wl.batch) for h in range(wl.num_kv_heads)]
    idx = rng.choice(len(all_units), size=min(n, len(all_units)), replace=False)
    picked = [all_units[i] for i in sorted(idx)]
    # always include the first and last unit (address arithmetic at both ends)
    for u in (all_units[0], all_units[-1]):
        if u not in picked:
            picked.append(u)
    return picked


def gather_units(out, lse, wl, units):
    G = wl.group
    got = np.stack([out[b, h * G:(h + 1) * G] for b, h in units])
    got_lse = np.stack([lse[b, h * G:(h + 1) * G] for b, h in units])
    return got, got_lse


def ragged_workload(dtype="bf16", B=8, Hkv=2, G=4, nb=1000, w=300, r=64, sigma=1.0, theta=5e5,
                    context=32768, index=95):
    """A small workload for ragged and paged tests: capacities nb, w."""
    return dataclasses.replace(
        synth.get_workload("c2"), name="ragged", index=index, batch=B, num_q_heads=Hkv * G,
        num_kv_heads=Hkv, num_beacons=nb, raw_window=w, ranks=(r,), dtype=dtype, sigma=sigma,
        rope_theta=theta, context=context)


def ragged_edge_cases(nb, w):
    """Sequence index -> (live beacons, live raw rows): no rows, full (the
    new token is attended but not stored), beyond the capacity (clamped),
    one row."""
    return {0: (0, 0), 1: (nb, w), 2: (nb + 7, -5), 3: (1, 1)}


def plant_counters(ws, units, value=3):
    """Write ``value`` into every unit's counters (they follow the
    workspace's 256-byte header, 16 uint32 per unit), as a call that did not
    run to its end could leave them."""
    ws[256:256 + 64 * units].view(torch.int32).view(units, 16)[:, :2] = value


def run_gpu_ragged(inp: synth.LayerInputs, step: synth.StepInputs, *, append: bool = True,
                   lengths: bool = True, num_splits: int = 0, device="cuda", flags: int = 0,
                   plant=None, status=None):
    """slimkv_decode_attn_ragged on ``inp`` (capacity-sized arrays) and
    ``step``.  The raw cache is cloned first (the call writes the new rows);
    returns (out, lse, K_raw, V_raw) on the host.  plant(ws): applied to the
    zero-filled workspace before the call; status (a list): receives the
    workspace's status word after it."""
    wl = inp.workload
    g = inp.to(device)
    st = step.to(device)
    K, V = g.K_raw.clone(), g.V_raw.clone()
    prob = lda.problem_from_tensors(g.q, g.U_K, g.C_K, g.K_raw, U_V=g.U_V,
                                    rope_theta=wl.rope_theta, num_kv_heads=wl.num_kv_heads,
                                    scale=wl.scale, num_splits=num_splits, flags=flags)
    out, lse = lda.alloc_outputs(prob, device)
    ws = lda.alloc_workspace(prob, lda.SLIMKV_OP_LATENT_RAGGED, device)
    if plant is not None:
        plant(ws)
    lda.slimkv_decode_attn_ragged(prob, g.q, g.q_pos, g.U_K, g.U_V, g.C_K, g.C_V, K, V,
                                  st.num_beacons if lengths else None,
                                  st.raw_len if lengths else None,
                                  st.k_new if append else None, st.v_new if append else None,
                                  out, lse, ws)
    torch.cuda.synchronize()
    if status is not None:
        status.append(lda.slimkv_workspace_status(ws))
    return (out.double().cpu().numpy(), lse.double().cpu().numpy(), K.cpu(), V.cpu())


def oracle_ragged(inp: synth.LayerInputs, step: synth.StepInputs, *, append: bool = True,
                  lengths: bool = True, units=None):
    """oracle.decode_ragged on the whole layer (or the listed units)."""
    wl = inp.workload
    st = synth.to_numpy_storage
    nb, w = inp.num_beacons, inp.raw_window
    return oracle.decode_ragged(
        st(inp.q), st(inp.q_pos), st(inp.U_K), st(inp.U_V), st(inp.C_K) if nb else None,
        st(inp.C_V) if nb else None, st(inp.K_raw) if w else None, st(inp.V_raw) if w else None,
        num_kv_heads=wl.num_kv_heads, scale=wl.scale, rope_theta=wl.rope_theta,
        num_beacons=st(step.num_beacons) if lengths else None,
        raw_len=st(step.raw_len) if lengths else None,
        k_new=st(step.k_new) if append else None, v_new=st(step.v_new) if append else None,
        units=units)


def oracle_ragged_units(inp: synth.LayerInputs, step: synth.StepInputs, units):
    """oracle.decode_ragged on sampled units, copying only each unit's slices.
    Returns {(b, h): (out [G, d], lse [G], k_app [d])}."""
    wl = inp.workload
    st = synth.to_numpy_storage
    res = {}
    for b, h in units:
        s = synth.unit_slices(inp, b, h)
        nb, w = s["C_K"].shape[2], s["K_raw"].shape[2]
        o, l, k = oracle.decode_ragged(
            s["q"], s["q_pos"], s["U_K"], s["U_V"], s["C_K"] if nb else None,
            s["C_V"] if nb else None, s["K_raw"] if w else None, s["V_raw"] if w else None,
            num_kv_heads=1, scale=wl.scale, rope_theta=wl.rope_theta,
            num_beacons=st(step.num_beacons[b:b + 1]), raw_len=st(step.raw_len[b:b + 1]),
            k_new=st(step.k_new[b:b + 1, h:h + 1]), v_new=st(step.v_new[b:b + 1, h:h + 1]))
        res[(b, h)] = (o[0], l[0], k[0, 0])
    return res


def storage_to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a bf16 or fp32 tensor."""
    return t.detach().cpu().to(torch.float64).numpy()


def _key_ulps(got, exp, dtype, where) -> int:
    """Elements of a stored key that differ from the oracle's (each by at
    most one ulp of the storage dtype, asserted)."""
    diff = got != exp
    if diff.any():
        ulp = np.abs(np.spacing(exp.astype(np.float32)).astype(np.float64))
        if dtype == torch.bfloat16:
            ulp = ulp * 65536.0
        assert np.all(np.abs(got - exp)[diff] <= ulp[diff] * 1.0001), \
            f"stored key of {where} off by more than one ulp"
    return int(diff.sum())


def assert_new_rows(K_after, V_after, K_before, V_before, step, k_app, units=None):
    """The call wrote exactly the new token's rows (row raw_len[b] of each
    unit whose window has room): keys equal the oracle's rotated, rounded
    key -- bit for bit, up to a rare one-ulp difference where the fp64
    rotation lands on a rounding tie (counted, at most 1 in 10^4) -- and
    values equal v_new; every other row is untouched."""
    Ka, Va = storage_to_f64(K_after), storage_to_f64(V_after)
    Kb, Vb = storage_to_f64(K_before), storage_to_f64(V_before)
    vnew = storage_to_f64(step.v_new)
    B, Hkv, wcap, d = Ka.shape
    mask = np.zeros((B, Hkv, wcap), dtype=bool)
    raw_len = step.raw_len.cpu().numpy()
    units = units or [(b, h) for b in range(B) for h in range(Hkv)]
    off_by_ulp = compared = 0
    for b, h in units:
        w = int(np.clip(raw_len[b], 0, wcap))
        if w >= wcap:
            continue
        mask[b, h, w] = True
        exp = k_app[(b, h)] if isinstance(k_app, dict) else k_app[b, h]
        off_by_ulp += _key_ulps(Ka[b, h, w], exp, K_after.dtype, (b, h))
        compared += d
        assert np.array_equal(Va[b, h, w], vnew[b, h]), f"stored value of ({b}, {h})"
    assert off_by_ulp <= max(1, compared // 10000), f"{off_by_ulp} of {compared} key elements"
    keep = ~mask
    if units is not None:
        sel = np.zeros((B, Hkv), dtype=bool)
        for b, h in units:
            sel[b, h] = True
        keep &= sel[:, :, None]
    assert np.array_equal(Ka[keep], Kb[keep]) and np.array_equal(Va[keep], Vb[keep]), \
        "rows other than the new token's were written"
    print(f"[parity] new rows: {int(mask.sum())} written, {off_by_ulp} key elements one ulp off",
          flush=True)



def run_gpu_paged(inp: synth.LayerInputs, step: synth.StepInputs, pc: synth.PagedCache, *,
                  append: bool = True, lengths: bool = True, num_splits: int = 0,
                  beacon_table=None, raw_table=None, device="cuda"):
    """slimkv_decode_attn_paged on ``pc`` (the pages of ``inp``'s capacity
    arrays) and ``step``; tables default to pc's.  The raw pools are cloned
    first (the call writes the new rows); returns (out, lse, K pool, V pool)
    on the host."""
    wl = inp.workload
    g = inp.to(device)
    st = step.to(device)
    ncap, wcap = inp.num_beacons, inp.raw_window
    bt = (pc.beacon_table if beacon_table is None else beacon_table).to(device)
    rt = (pc.raw_table if raw_table is None else raw_table).to(device)
    CK, CV = pc.C_K.to(device), pc.C_V.to(device)
    K, V = pc.K_raw.to(device).clone(), pc.V_raw.to(device).clone()
    prob = lda.problem_from_tensors(g.q, g.U_K, g.C_K, g.K_raw, U_V=g.U_V,
                                    rope_theta=wl.rope_theta, num_kv_heads=wl.num_kv_heads,
                                    scale=wl.scale, num_splits=num_splits)
    pages = lda.make_pages(page_rows=pc.page_rows, beacon_table=bt if ncap else None,
                           raw_table=rt if wcap else None, beacon_pages=pc.beacon_pages,
                           raw_pages=pc.raw_pages)
    out, lse = lda.alloc_outputs(prob, device)
    ws = lda.alloc_workspace(prob, lda.SLIMKV_OP_LATENT_RAGGED, device)
    lda.slimkv_decode_attn_paged(prob, pages, g.q, g.q_pos, g.U_K, g.U_V,
                                 CK if ncap else None, CV if ncap else None,
                                 K if wcap else None, V if wcap else None,
                                 st.num_beacons if lengths else None,
                                 st.raw_len if lengths else None,
                                 st.k_new if append else None, st.v_new if append else None,
                                 out, lse, ws)
    torch.cuda.synchronize()
    return (out.double().cpu().numpy(), lse.double().cpu().numpy(), K.cpu(), V.cpu())


def storage_bits(t: torch.Tensor) -> np.ndarray:
    """The bit patterns of a bf16 or fp32 tensor (NaNs compare equal)."""
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy()


def assert_paged_writes(K_after, V_after, pc: synth.PagedCache, step, k_app, wcap: int,
                        raw_table=None, units=None):
    """The paged call wrote exactly the new token's rows -- row raw_len[b] of
    each unit whose window has room, in the page the raw table gives for it
    (none if that id is out of range) -- with the oracle's key (as in
    assert_new_rows) and v_new, checked for ``units`` (default all); every
    other element of both pools, NaN fillers of unused rows and pages
    included, keeps its bits.  k_app None: no new token, nothing written."""
    table = (pc.raw_table if raw_table is None else raw_table).cpu().numpy()
    PR = pc.page_rows
    Ka, Va = storage_to_f64(K_after), storage_to_f64(V_after)
    vnew = storage_to_f64(step.v_new)
    raw_len = step.raw_len.cpu().numpy()
    B, Hkv = vnew.shape[0], vnew.shape[1]
    check = set(units or [(b, h) for b in range(B) for h in range(Hkv)])
    mask = np.zeros(K_after.shape[:3], dtype=bool)
    off_by_ulp = compared = 0
    for b in range(B if k_app is not None else 0):
        w = int(np.clip(raw_len[b], 0, wcap))
        if w >= wcap:
            continue
        pid = int(table[b, w // PR])
        if not 0 <= pid < K_after.shape[0]:
            continue
        r = w % PR
        mask[pid, :, r] = True
        for h in range(Hkv):
            if (b, h) in check:
                exp = k_app[(b, h)] if isinstance(k_app, dict) else k_app[b, h]
                off_by_ulp += _key_ulps(Ka[pid, h, r], exp, K_after.dtype, (b, h))
                compared += Ka.shape[-1]
                assert np.array_equal(Va[pid, h, r], vnew[b, h]), f"stored value of ({b}, {h})"
    assert off_by_ulp <= max(1, compared // 10000), f"{off_by_ulp} of {compared} key elements"
    keep = ~mask
    assert np.array_equal(storage_bits(K_after)[keep], storage_bits(pc.K_raw)[keep]), \
        "K pool: other rows written"
    assert np.array_equal(storage_bits(V_after)[keep], storage_bits(pc.V_raw)[keep]), \
        "V pool: other rows written"
    print(f"[parity] paged new rows: {int(mask.sum())} written, {off_by_ulp} key elements one "
          f"ulp off", flush=True)


def run_gpu_chunk(inp: synth.LayerInputs, ch: synth.ChunkInputs, *, append: bool = True,
                  lengths: bool = True, num_splits: int = 0, device="cuda", flags: int = 0,
                  plant=None, status=None):
    """slimkv_decode_attn_chunk on ``inp`` (capacity-sized arrays) and the
    chunk ``ch``; the raw cache is cloned first.  Returns (out [B, Q, H_q, d],
    lse [B, Q, H_q], K_raw, V_raw) on the host.  plant, status: as for
    run_gpu_ragged."""
    wl = inp.workload
    g = inp.to(device)
    c = ch.to(device)
    Q = ch.num_tokens
    K, V = g.K_raw.clone(), g.V_raw.clone()
    prob = lda.problem_from_tensors(g.q, g.U_K, g.C_K, g.K_raw, U_V=g.U_V,
                                    rope_theta=wl.rope_theta, num_kv_heads=wl.num_kv_heads,
                                    scale=wl.scale, num_splits=num_splits, flags=flags)
    B, Hq, d = g.q.shape
    out = torch.empty((B, Q, Hq, d), dtype=torch.float32, device=device)
    lse = torch.empty((B, Q, Hq), dtype=torch.float32, device=device)
    ws = torch.zeros(lda.slimkv_chunk_workspace_bytes(prob, Q), dtype=torch.uint8, device=device)
    if plant is not None:
        plant(ws)
    lda.slimkv_decode_attn_chunk(prob, Q, c.q, g.q_pos, g.U_K, g.U_V, g.C_K, g.C_V, K, V,
                                 c.num_beacons if lengths else None,
                                 c.raw_len if lengths else None,
                                 c.k_new if append else None, c.v_new if append else None,
                                 out, lse, ws)
    torch.cuda.synchronize()
    if status is not None:
        status.append(lda.slimkv_workspace_status(ws))
    return out.double().cpu().numpy(), lse.double().cpu().numpy(), K.cpu(), V.cpu()


def run_gpu_chunk_paged(inp: synth.LayerInputs, ch: synth.ChunkInputs, pc: synth.PagedCache, *,
                        append: bool = True, lengths: bool = True, num_splits: int = 0,
                        raw_table=None, device="cuda"):
    """slimkv_decode_attn_chunk_paged on ``pc`` (the pages of ``inp``'s
    capacity arrays) and the chunk ``ch``; the raw pools are cloned first.
    Returns (out [B, Q, H_q, d], lse [B, Q, H_q], K pool, V pool) on the host."""
    wl = inp.workload
    g = inp.to(device)
    c = ch.to(device)
    Q = ch.num_tokens
    ncap, wcap = inp.num_beacons, inp.raw_window
    # the tables stay referenced until the call: the struct keeps raw pointers
    bt = pc.beacon_table.to(device)
    rt = (pc.raw_table if raw_table is None else raw_table).to(device)
    CK, CV = pc.C_K.to(device), pc.C_V.to(device)
    K, V = pc.K_raw.to(device).clone(), pc.V_raw.to(device).clone()
    prob = lda.problem_from_tensors(g.q, g.U_K, g.C_K, g.K_raw, U_V=g.U_V,
                                    rope_theta=wl.rope_theta, num_kv_heads=wl.num_kv_heads,
                                    scale=wl.scale, num_splits=num_splits)
    pages = lda.make_pages(page_rows=pc.page_rows, beacon_table=bt if ncap else None,
                           raw_table=rt if wcap else None, beacon_pages=pc.beacon_pages,
                           raw_pages=pc.raw_pages)
    B, Hq, d = g.q.shape
    out = torch.empty((B, Q, Hq, d), dtype=torch.float32, device=device)
    lse = torch.empty((B, Q, Hq), dtype=torch.float32, device=device)
    ws = torch.zeros(lda.slimkv_chunk_workspace_bytes(prob, Q), dtype=torch.uint8, device=device)
    lda.slimkv_decode_attn_chunk_paged(prob, pages, Q, c.q, g.q_pos, g.U_K, g.U_V,
                                       CK if ncap else None, CV if ncap else None,
                                       K if wcap else None, V if wcap else None,
                                       c.num_beacons if lengths else None,
                                       c.raw_len if lengths else None,
                                       c.k_new if append else None, c.v_new if append else None,
                                       out, lse, ws)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), lse.double().cpu().numpy(), K.cpu(), V.cpu()


def assert_chunk_paged_writes(K_after, V_after, pc: synth.PagedCache, ch: synth.ChunkInputs, k_app,
                              wcap: int, raw_table=None, units=None):
    """The paged chunk call wrote exactly its tokens' rows -- raw row w_b + u
    for every token u with w_b + u below the capacity, in the page the raw
    table gives for that row (none if the id is out of range) -- with the
    oracle's keys (as in assert_new_rows; k_app [B, Q, H_kv, d] or
    {(b, h): [Q, d]}) and v_new, checked for ``units`` (default all); every
    other element of both pools, NaN fillers included, keeps its bits.
    k_app None: no tokens, nothing written."""
    table = (pc.raw_table if raw_table is None else raw_table).cpu().numpy()
    PR = pc.page_rows
    Ka, Va = storage_to_f64(K_after), storage_to_f64(V_after)
    vnew = storage_to_f64(ch.v_new)
    raw_len = ch.raw_len.cpu().numpy()
    B, Q, Hkv = vnew.shape[0], vnew.shape[1], vnew.shape[2]
    check = set(units or [(b, h) for b in range(B) for h in range(Hkv)])
    mask = np.zeros(K_after.shape[:3], dtype=bool)
    off_by_ulp = compared = 0
    for b in range(B if k_app is not None else 0):
        w = int(np.clip(raw_len[b], 0, wcap))
        for u in range(Q):
            if w + u >= wcap:
                break
            pid = int(table[b, (w + u) // PR])
            if not 0 <= pid < K_after.shape[0]:
                continue
            r = (w + u) % PR
            mask[pid, :, r] = True
            for h in range(Hkv):
                if (b, h) in check:
                    exp = k_app[(b, h)][u] if isinstance(k_app, dict) else k_app[b, u, h]
                    off_by_ulp += _key_ulps(Ka[pid, h, r], exp, K_after.dtype, (b, h, u))
                    compared += Ka.shape[-1]
                    assert np.array_equal(Va[pid, h, r], vnew[b, u, h]), f"value ({b}, {h}, {u})"
    assert off_by_ulp <= max(1, compared // 10000), f"{off_by_ulp} of {compared} key elements"
    keep = ~mask
    assert np.array_equal(storage_bits(K_after)[keep], storage_bits(pc.K_raw)[keep]), \
        "K pool: other rows written"
    assert np.array_equal(storage_bits(V_after)[keep], storage_bits(pc.V_raw)[keep]), \
        "V pool: other rows written"
    print(f"[parity] paged chunk rows: {int(mask.sum())} written, {off_by_ulp} key elements one "
          f"ulp off", flush=True)


def oracle_chunk(inp: synth.LayerInputs, ch: synth.ChunkInputs, *, append: bool = True,
                 lengths: bool = True, units=None):
    """oracle.decode_chunk on the whole layer (or the listed units)."""
    wl = inp.workload
    st = synth.to_numpy_storage
    nb, w = inp.num_beacons, inp.raw_window
    return oracle.decode_chunk(
        st(ch.q), st(inp.q_pos), st(inp.U_K), st(inp.U_V), st(inp.C_K) if nb else None,
        st(inp.C_V) if nb else None, st(inp.K_raw) if w else None, st(inp.V_raw) if w else None,
        num_kv_heads=wl.num_kv_heads, scale=wl.scale, rope_theta=wl.rope_theta,
        num_beacons=st(ch.num_beacons) if lengths else None,
        raw_len=st(ch.raw_len) if lengths else None,
        k_new=st(ch.k_new) if append else None, v_new=st(ch.v_new) if append else None,
        units=units)


def oracle_chunk_units(inp: synth.LayerInputs, ch: synth.ChunkInputs, units):
    """oracle.decode_chunk on sampled units, copying only each unit's slices.
    Returns {(b, h): (out [Q, G, d], lse [Q, G], k_app [Q, d])}."""
    wl = inp.workload
    st = synth.to_numpy_storage
    G = wl.group
    res = {}
    for b, h in units:
        hs = slice(h * G, (h + 1) * G)
        nb, w = inp.num_beacons, inp.raw_window
        out, lse, k_app = oracle.decode_chunk(
            st(ch.q[b:b + 1, :, hs]), st(inp.q_pos[b:b + 1]), st(inp.U_K[h:h + 1]),
            st(inp.U_V[h:h + 1]), st(inp.C_K[b:b + 1, h:h + 1]) if nb else None,
            st(inp.C_V[b:b + 1, h:h + 1]) if nb else None,
            st(inp.K_raw[b:b + 1, h:h + 1]) if w else None,
            st(inp.V_raw[b:b + 1, h:h + 1]) if w else None,
            num_kv_heads=1, scale=wl.scale, rope_theta=wl.rope_theta,
            num_beacons=st(ch.num_beacons[b:b + 1]), raw_len=st(ch.raw_len[b:b + 1]),
            k_new=st(ch.k_new[b:b + 1, :, h:h + 1]), v_new=st(ch.v_new[b:b + 1, :, h:h + 1]))
        res[(b, h)] = (out[0], lse[0], k_app[0, :, 0])
    return res


def assert_chunk_rows(K_after, V_after, K_before, V_before, ch: synth.ChunkInputs, k_app,
                      units=None):
    """The chunk call wrote exactly its tokens' rows -- raw row w_b + u for
    every token u with w_b + u below the capacity -- with the oracle's keys
    (as in assert_new_rows; k_app [B, Q, H_kv, d] or {(b, h): [Q, d]}) and
    v_new, checked for ``units`` (default all); every other row keeps its
    bits.  k_app None: no tokens, nothing written."""
    Ka, Va = storage_to_f64(K_after), storage_to_f64(V_after)
    vnew = storage_to_f64(ch.v_new)
    B, Hkv, wcap, d = Ka.shape
    Q = ch.num_tokens
    raw_len = ch.raw_len.cpu().numpy()
    check = set(units or [(b, h) for b in range(B) for h in range(Hkv)])
    mask = np.zeros((B, Hkv, wcap), dtype=bool)
    off_by_ulp = compared = 0
    for b in range(B if k_app is not None else 0):
        w = int(np.clip(raw_len[b], 0, wcap))
        for u in range(Q):
            if w + u >= wcap:
                break
            mask[b, :, w + u] = True
            for h in range(Hkv):
                if (b, h) in check:
                    exp = k_app[(b, h)][u] if isinstance(k_app, dict) else k_app[b, u, h]
                    off_by_ulp += _key_ulps(Ka[b, h, w + u], exp, K_after.dtype, (b, h, u))
                    compared += d
                    assert np.array_equal(Va[b, h, w + u], vnew[b, u, h]), f"value ({b}, {h}, {u})"
    assert off_by_ulp <= max(1, compared // 10000), f"{off_by_ulp} of {compared} key elements"
    keep = ~mask
    assert np.array_equal(storage_bits(K_after)[keep], storage_bits(K_before)[keep]), \
        "K_raw: other rows written"
    assert np.array_equal(storage_bits(V_after)[keep], storage_bits(V_before)[keep]), \
        "V_raw: other rows written"
    print(f"[parity] chunk rows: {int(mask.sum())} written, {off_by_ulp} key elements one ulp off",
          flush=True)


def run_gpu_alibi(inp: synth.LayerInputs, slopes: np.ndarray, first: int, stride: int, *,
                  num_splits: int = 0, device="cuda"):
    """slimkv_decode_attn_alibi on ``inp`` with per-query-head slopes and
    beacon j at first + j * stride; returns (out, lse) on the host."""
    wl = inp.workload
    g = inp.to(device)
    prob = lda.problem_from_tensors(g.q, g.U_K, g.C_K, g.K_raw, U_V=g.U_V,
                                    rope_theta=wl.rope_theta, num_kv_heads=wl.num_kv_heads,
                                    scale=wl.scale, num_splits=num_splits)
    out, lse = lda.alloc_outputs(prob, device)
    ws = lda.alloc_workspace(prob, lda.SLIMKV_OP_LATENT, device)
    sl = torch.as_tensor(np.asarray(slopes, dtype=np.float32), device=device)
    nb, w = inp.num_beacons, inp.raw_window
    lda.slimkv_decode_attn_alibi(prob, g.q, g.q_pos, g.U_K if nb else None, g.U_V if nb else None,
                                 g.C_K if nb else None, g.C_V if nb else None,
                                 g.K_raw if w else None, g.V_raw if w else None, sl, first, stride,
                                 out, lse, ws)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), lse.double().cpu().numpy()


def oracle_alibi(inp: synth.LayerInputs, slopes: np.ndarray, first: int, stride: int, units=None):
    """oracle.decode_alibi on the whole layer (or the listed units); the
    slopes are taken as the fp32 values the GPU receives."""
    wl = inp.workload
    st = synth.to_numpy_storage
    nb, w = inp.num_beacons, inp.raw_window
    bpos = (first + stride * np.arange(nb)).astype(np.int32)
    return oracle.decode_alibi(
        st(inp.q), st(inp.q_pos), st(inp.U_K), st(inp.U_V), st(inp.C_K) if nb else None,
        st(inp.C_V) if nb else None, st(inp.K_raw) if w else None, st(inp.V_raw) if w else None,
        beacon_pos=bpos, slopes=np.asarray(slopes, dtype=np.float32).astype(np.float64),
        num_kv_heads=wl.num_kv_heads, scale=wl.scale, units=units)
