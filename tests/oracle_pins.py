"""Checks that pin the fp64 oracle to things other than itself.

Each ``pin_*`` function raises AssertionError when the oracle built at
``library`` disagrees with an independent statement of what the method
computes (page "Can SlimKV compress KV cache jointly across tokens and
features", section "Latent-space attention removes the rebuild step"):

* reconstruct-then-attend: building full beacon keys C_K U_K^T and values
  C_V U_V^T and running ordinary attention (torch's fp64 SDPA) must give the
  same result as the latent path -- the identity the section rests on;
* a raw-only window is ordinary rotary GQA attention, with the rotation
  written independently as complex multiplication;
* with an identity basis and no raw window, beacon keys enter unrotated;
* rotary scores depend only on relative position;
* closed forms of the softmax (zero query, one key, two keys);
* invariants: weights sum to one, orthogonal re-basing of a latent space,
  row permutations.

The same functions run against deliberately broken copies of the oracle
(tests/test_oracle_mutants.py) to show that a plausible mistake fails one.
"""

from __future__ import annotations

import math

import numpy as np
import torch

import oracle

TOL = 1e-11


def _ortho(rng, d, r):
    a = rng.standard_normal((d, r))
    qm, rm = np.linalg.qr(a)
    return qm * np.sign(np.diag(rm))


def rope_complex(x: np.ndarray, pos, theta: float) -> np.ndarray:
    """Rotary embedding as complex multiplication: pair (i, i + d/2) is the
    complex number x_i + 1j x_{i+d/2}, turned by angle pos * theta**(-2i/d).
    ``pos`` broadcasts against the leading axes of x."""
    d = x.shape[-1]
    half = d // 2
    freqs = np.exp(-(2.0 * np.arange(half) / d) * math.log(theta))
    ang = np.asarray(pos, dtype=np.float64)[..., None] * freqs
    z = (x[..., :half] + 1j * x[..., half:]) * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag], axis=-1)


def random_problem(seed, *, B=1, Hkv=1, G=4, d=16, nb=5, rk=4, rv=6, w=3, theta=10000.0,
                   q_pos=None, sigma=1.0):
    rng = np.random.default_rng(seed)
    Hq = Hkv * G
    qp = np.full(B, w + 7 if q_pos is None else q_pos, dtype=np.int32)
    raw_pos = qp[:, None] - w + 1 + np.arange(w)[None, :]  # [B, W]
    k_pre = sigma * rng.standard_normal((B, Hkv, w, d))
    return dict(
        q=sigma * rng.standard_normal((B, Hq, d)),
        q_pos=qp,
        U_K=np.stack([_ortho(rng, d, rk) for _ in range(Hkv)]),
        U_V=np.stack([_ortho(rng, d, rv) for _ in range(Hkv)]),
        C_K=sigma * rng.standard_normal((B, Hkv, nb, rk)),
        C_V=sigma * rng.standard_normal((B, Hkv, nb, rv)),
        K_pre=k_pre,
        K_raw=rope_complex(k_pre, raw_pos[:, None, :], theta),
        V_raw=sigma * rng.standard_normal((B, Hkv, w, d)),
        theta=theta,
        scale=1.0 / math.sqrt(d),
        num_kv_heads=Hkv,
    )


def run_oracle(p, library, beacon_pos=None, **over):
    args = dict(p)
    args.update(over)
    nb = args["C_K"].shape[2]
    w = args["K_raw"].shape[2]
    return oracle.decode(
        args["q"], args["q_pos"], args["U_K"], args["U_V"],
        args["C_K"] if nb else None, args["C_V"] if nb else None,
        args["K_raw"] if w else None, args["V_raw"] if w else None,
        num_kv_heads=args["num_kv_heads"], scale=args["scale"], rope_theta=args["theta"],
        library=library, beacon_pos=beacon_pos)


def sdpa_reference(q_rot, K, V, scale, G):
    """Ordinary attention of one query per head; K, V: [B, H_kv, n, d]."""
    qt = torch.from_numpy(q_rot)[:, :, None, :]  # [B, Hq, 1, d]
    kt = torch.from_numpy(np.ascontiguousarray(K)).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(np.ascontiguousarray(V)).repeat_interleave(G, dim=1)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    scores = scale * torch.matmul(qt, kt.transpose(-1, -2).contiguous())[:, :, 0, :]
    lse = torch.logsumexp(scores, dim=-1)
    return out[:, :, 0, :].numpy(), lse.numpy()


def reconstruct_reference(p):
    G = p["q"].shape[1] // p["num_kv_heads"]
    q_rot = rope_complex(p["q"], p["q_pos"][:, None], p["theta"])
    kb = np.einsum("bhjr,hdr->bhjd", p["C_K"], p["U_K"])
    vb = np.einsum("bhjr,hdr->bhjd", p["C_V"], p["U_V"])
    K = np.concatenate([kb, p["K_raw"]], axis=2)
    V = np.concatenate([vb, p["V_raw"]], axis=2)
    return sdpa_reference(q_rot, K, V, p["scale"], G)


def _close(a, b, tol=TOL, what=""):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b))))
    ref = max(1.0, float(np.max(np.abs(b))))
    assert err <= tol * ref, f"{what}: max abs error {err:.3e} (tolerance {tol * ref:.1e})"


SHAPES = [
    dict(B=1, Hkv=1, G=1, d=8, nb=1, rk=2, rv=3, w=0),
    dict(B=2, Hkv=2, G=4, d=16, nb=17, rk=4, rv=8, w=3),
    dict(B=1, Hkv=3, G=5, d=16, nb=0, rk=4, rv=4, w=17),
    dict(B=2, Hkv=1, G=4, d=128, nb=33, rk=32, rv=48, w=1),
    dict(B=1, Hkv=2, G=2, d=128, nb=3, rk=64, rv=16, w=17, theta=500000.0, q_pos=131071),
]


def pin_reconstruct_identity(library):
    for i, shape in enumerate(SHAPES):
        p = random_problem(100 + i, **shape)
        out, lse = run_oracle(p, library)
        ref_out, ref_lse = reconstruct_reference(p)
        _close(out, ref_out, what=f"out, shape {shape}")
        _close(lse, ref_lse, what=f"lse, shape {shape}")


def pin_raw_only_rope_gqa(library):
    p = random_problem(7, B=2, Hkv=2, G=4, d=128, nb=0, rk=8, rv=8, w=29, theta=500000.0,
                       q_pos=32767)
    out, lse = run_oracle(p, library)
    q_rot = rope_complex(p["q"], p["q_pos"][:, None], p["theta"])
    ref_out, ref_lse = sdpa_reference(q_rot, p["K_raw"], p["V_raw"], p["scale"], 4)
    _close(out, ref_out, what="raw-only out")
    _close(lse, ref_lse, what="raw-only lse")


def pin_beacon_keys_unrotated(library):
    d = 16
    p = random_problem(8, B=1, Hkv=2, G=2, d=d, nb=9, rk=d, rv=d, w=0, q_pos=12345)
    eye = np.stack([np.eye(d), np.eye(d)])
    p["U_K"], p["U_V"] = eye, eye
    out, lse = run_oracle(p, library)
    q_rot = rope_complex(p["q"], p["q_pos"][:, None], p["theta"])
    ref_out, ref_lse = sdpa_reference(q_rot, p["C_K"], p["C_V"], p["scale"], 2)
    _close(out, ref_out, what="beacon-only out")
    _close(lse, ref_lse, what="beacon-only lse")


def pin_relative_position(library):
    """Raw-only window: shifting the query and every raw key by the same
    offset leaves the result unchanged; shifting only the query changes it.
    (Beacon keys carry no rotation, so with beacons present the property
    does not hold and is not tested here.)"""
    p = random_problem(9, B=1, Hkv=1, G=4, d=32, nb=0, rk=8, rv=8, w=6, q_pos=50)
    out0, lse0 = run_oracle(p, library)
    for shift in (1, 1000, 100000):
        qp = p["q_pos"] + shift
        raw_pos = qp[:, None] - 6 + 1 + np.arange(6)[None, :]
        k = rope_complex(p["K_pre"], raw_pos[:, None, :], p["theta"])
        out1, lse1 = run_oracle(p, library, q_pos=qp.astype(np.int32), K_raw=k)
        _close(out1, out0, tol=1e-9, what=f"shift {shift}")
        _close(lse1, lse0, tol=1e-9, what=f"shift {shift}")
    out2, _ = run_oracle(p, library, q_pos=(p["q_pos"] + 3).astype(np.int32))
    assert np.max(np.abs(out2 - out0)) > 1e-6, "query position has no effect"


def pin_position_zero(library):
    p = random_problem(10, B=1, Hkv=1, G=2, d=16, nb=0, rk=4, rv=4, w=5, q_pos=0)
    out, _ = run_oracle(p, library)
    ref, _ = sdpa_reference(p["q"], p["K_raw"], p["V_raw"], p["scale"], 2)
    _close(out, ref, what="position 0")


def pin_constant_values(library):
    """Every value row equal to the all-ones vector => out is exactly 1."""
    d, rv = 16, 4
    p = random_problem(11, B=2, Hkv=1, G=3, d=d, nb=7, rk=4, rv=rv, w=5)
    rng = np.random.default_rng(5)
    basis = np.concatenate([np.ones((d, 1)) / math.sqrt(d), rng.standard_normal((d, rv - 1))], 1)
    uv, rm = np.linalg.qr(basis)
    uv = uv * np.sign(np.diag(rm))
    cv = np.zeros_like(p["C_V"])
    cv[..., 0] = math.sqrt(d)
    out, _ = run_oracle(p, library, U_V=uv[None], C_V=cv, V_raw=np.ones_like(p["V_raw"]))
    _close(out, np.ones_like(out), tol=1e-12, what="constant values")


def pin_rebasing(library):
    """(U_K R, C_K R) and (U_V S, C_V S) with orthogonal R, S leave out unchanged."""
    p = random_problem(12, B=1, Hkv=2, G=2, d=16, nb=6, rk=5, rv=7, w=2)
    out0, lse0 = run_oracle(p, library)
    rng = np.random.default_rng(3)
    R = _ortho(rng, 5, 5)
    S = _ortho(rng, 7, 7)
    out1, lse1 = run_oracle(p, library, U_K=p["U_K"] @ R, C_K=p["C_K"] @ R,
                            U_V=p["U_V"] @ S, C_V=p["C_V"] @ S)
    _close(out1, out0, what="re-based out")
    _close(lse1, lse0, what="re-based lse")


def pin_permutations(library):
    p = random_problem(13, B=1, Hkv=1, G=4, d=16, nb=8, rk=4, rv=4, w=6)
    out0, _ = run_oracle(p, library)
    pb = np.random.default_rng(1).permutation(8)
    pr = np.random.default_rng(2).permutation(6)
    out1, _ = run_oracle(p, library, C_K=p["C_K"][:, :, pb], C_V=p["C_V"][:, :, pb],
                         K_raw=p["K_raw"][:, :, pr], V_raw=p["V_raw"][:, :, pr])
    _close(out1, out0, what="permuted rows")


def pin_closed_forms(library):
    # zero query: uniform weights, out = mean of all value rows, lse = log(n)
    p = random_problem(14, B=1, Hkv=1, G=2, d=16, nb=5, rk=4, rv=6, w=3)
    zq = np.zeros_like(p["q"])
    out, lse = run_oracle(p, library, q=zq)
    vals = np.concatenate([p["C_V"][0, 0] @ p["U_V"][0].T, p["V_raw"][0, 0]], axis=0)
    _close(out[0], np.broadcast_to(vals.mean(axis=0), out[0].shape), what="zero query")
    _close(lse, np.full_like(lse, math.log(8)), what="zero-query lse")
    # one raw key: out is that value row, lse is its score
    p1 = random_problem(15, B=1, Hkv=1, G=1, d=16, nb=0, rk=4, rv=4, w=1)
    out, lse = run_oracle(p1, library)
    _close(out[0, 0], p1["V_raw"][0, 0, 0], what="single key")
    q_rot = rope_complex(p1["q"], p1["q_pos"][:, None], p1["theta"])
    s = p1["scale"] * float(q_rot[0, 0] @ p1["K_raw"][0, 0, 0])
    _close(lse[0, 0], s, what="single-key lse")
    # one beacon and one raw key: weight of the beacon is sigmoid(s_b - s_r)
    p2 = random_problem(16, B=1, Hkv=1, G=1, d=16, nb=1, rk=16, rv=16, w=1)
    p2["U_K"] = np.eye(16)[None]
    p2["U_V"] = np.eye(16)[None]
    out, _ = run_oracle(p2, library)
    q_rot = rope_complex(p2["q"], p2["q_pos"][:, None], p2["theta"])[0, 0]
    sb = p2["scale"] * float(q_rot @ p2["C_K"][0, 0, 0])
    sr = p2["scale"] * float(q_rot @ p2["K_raw"][0, 0, 0])
    a = 1.0 / (1.0 + math.exp(-(sb - sr)))
    _close(out[0, 0], a * p2["C_V"][0, 0, 0] + (1 - a) * p2["V_raw"][0, 0, 0], what="two keys")


# ---------------------------------------------------------------------------
# Ragged batches and the decode step's new token (oracle.decode_ragged).  A
# serving step attends each sequence over its own live rows of capacity-sized
# arrays, after rotating the new token's key at the query position and adding
# it as one more raw row; the references below rebuild each sequence's rows
# and run ordinary attention on them.


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest bfloat16 value (ties to even), on the
    IEEE bit pattern: keep 1 + 8 + 7 bits of 1 + 11 + 52."""
    bits = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)
    drop = np.uint64(52 - 7)
    half = np.uint64(1) << (drop - np.uint64(1))
    keep_lsb = (bits >> drop) & np.uint64(1)
    rounded = (bits + half - np.uint64(1) + keep_lsb) >> drop << drop
    return rounded.view(np.float64)


def ragged_problem(seed, *, B=4, Hkv=2, G=2, d=16, ncap=9, rk=4, rv=6, wcap=7, theta=10000.0,
                   q_pos=None, append=True):
    p = random_problem(seed, B=B, Hkv=Hkv, G=G, d=d, nb=ncap, rk=rk, rv=rv, w=wcap, theta=theta,
                       q_pos=q_pos)
    rng = np.random.default_rng(seed + 1000)
    p["num_beacons"] = rng.integers(0, ncap + 1, size=B).astype(np.int32)
    p["raw_len"] = rng.integers(0, wcap + 1, size=B).astype(np.int32)
    if append:
        p["k_new"] = rng.standard_normal((B, Hkv, d))
        p["v_new"] = rng.standard_normal((B, Hkv, d))
    return p


def run_ragged(p, library, **over):
    args = dict(p)
    args.update(over)
    ncap = args["C_K"].shape[2]
    wcap = args["K_raw"].shape[2]
    return oracle.decode_ragged(
        args["q"], args["q_pos"], args["U_K"], args["U_V"],
        args["C_K"] if ncap else None, args["C_V"] if ncap else None,
        args["K_raw"] if wcap else None, args["V_raw"] if wcap else None,
        num_kv_heads=args["num_kv_heads"], scale=args["scale"], rope_theta=args["theta"],
        num_beacons=args.get("num_beacons"), raw_len=args.get("raw_len"),
        k_new=args.get("k_new"), v_new=args.get("v_new"), library=library)


def ragged_reference(p, b):
    """Sequence b alone: its live beacon rows rebuilt to full keys and
    values, its live raw rows, and the new token (key rotated at q_pos[b])
    as the last row; ordinary attention over them.  Returns (out [H_q, d],
    lse [H_q]); a sequence without rows gives zeros and -inf."""
    Hkv = p["num_kv_heads"]
    G = p["q"].shape[1] // Hkv
    nbc = int(np.clip(p["num_beacons"][b], 0, p["C_K"].shape[2]))
    wc = int(np.clip(p["raw_len"][b], 0, p["K_raw"].shape[2]))
    kb = np.einsum("hjr,hdr->hjd", p["C_K"][b, :, :nbc], p["U_K"])
    vb = np.einsum("hjr,hdr->hjd", p["C_V"][b, :, :nbc], p["U_V"])
    K = [kb, p["K_raw"][b, :, :wc]]
    V = [vb, p["V_raw"][b, :, :wc]]
    if p.get("k_new") is not None:
        K.append(rope_complex(p["k_new"][b], np.full(Hkv, p["q_pos"][b]), p["theta"])[:, None, :])
        V.append(p["v_new"][b][:, None, :])
    K = np.concatenate(K, axis=1)[None]
    V = np.concatenate(V, axis=1)[None]
    if K.shape[2] == 0:
        d = p["q"].shape[2]
        return np.zeros((Hkv * G, d)), np.full(Hkv * G, -np.inf)
    q_rot = rope_complex(p["q"][b:b + 1], p["q_pos"][b:b + 1, None], p["theta"])
    out, lse = sdpa_reference(q_rot, K, V, p["scale"], G)
    return out[0], lse[0]


def pin_ragged_lengths(library):
    """Per-sequence live rows of capacity-sized arrays, without a new token;
    dead rows hold large values that must not leak in."""
    for seed, shape in ((40, dict(B=5, Hkv=2, G=2, d=16, ncap=9, rk=4, rv=6, wcap=7)),
                        (41, dict(B=3, Hkv=1, G=4, d=32, ncap=0, rk=4, rv=4, wcap=11)),
                        (42, dict(B=3, Hkv=2, G=1, d=16, ncap=13, rk=8, rv=4, wcap=0))):
        p = ragged_problem(seed, append=False, **shape)
        p["num_beacons"][0] = shape["ncap"]
        p["raw_len"][0] = shape["wcap"]
        if shape["B"] > 2:
            p["num_beacons"][1] = 0
            p["raw_len"][1] = 0
            # lengths outside [0, capacity] are clamped
            p["num_beacons"][2] = shape["ncap"] + 5
            p["raw_len"][2] = -3
        for name, n in (("C_K", "num_beacons"), ("C_V", "num_beacons"), ("K_raw", "raw_len"),
                        ("V_raw", "raw_len")):
            for b in range(shape["B"]):
                p[name][b, :, max(p[n][b], 0):] = 1e6
        out, lse, _ = run_ragged(p, library)
        for b in range(shape["B"]):
            ref_out, ref_lse = ragged_reference(p, b)
            _close(out[b], ref_out, what=f"ragged out, seq {b}, {shape}")
            if np.isinf(ref_lse).all():
                assert np.all(np.isneginf(lse[b])), "empty sequence lse"
            else:
                _close(lse[b], ref_lse, what=f"ragged lse, seq {b}, {shape}")


def pin_append_token(library):
    """The new token joins its sequence as a rotated raw row; its stored key
    is the rotation of k_new at the query position."""
    for seed, shape in ((43, dict(B=4, Hkv=2, G=2, d=16, ncap=6, rk=4, rv=4, wcap=5)),
                        (44, dict(B=2, Hkv=1, G=4, d=128, ncap=33, rk=32, rv=16, wcap=3,
                                  theta=500000.0, q_pos=131071))):
        p = ragged_problem(seed, **shape)
        p["raw_len"][0] = shape["wcap"]  # full window: attended, not storable
        out, lse, k_app = run_ragged(p, library)
        for b in range(shape["B"]):
            ref_out, ref_lse = ragged_reference(p, b)
            _close(out[b], ref_out, what=f"append out, seq {b}")
            _close(lse[b], ref_lse, what=f"append lse, seq {b}")
        ref_k = rope_complex(p["k_new"], p["q_pos"][:, None], p["theta"])
        _close(k_app, ref_k, tol=1e-10, what="rotated new key")


def pin_append_self_score(library):
    """A sequence holding only the new token: the output is its value and the
    log-sum-exp is its score, which is scale * q.k whatever the position
    (query and key turn by the same angle)."""
    for q_pos in (0, 77, 131071):
        p = ragged_problem(45, B=2, Hkv=2, G=3, d=32, ncap=4, rk=4, rv=4, wcap=3, q_pos=q_pos,
                           theta=500000.0)
        p["num_beacons"][:] = 0
        p["raw_len"][:] = 0
        out, lse, _ = run_ragged(p, library)
        for b in range(2):
            for hq in range(6):
                h = hq // 3
                _close(out[b, hq], p["v_new"][b, h], tol=1e-14, what="single-token out")
                s = p["scale"] * float(p["q"][b, hq] @ p["k_new"][b, h])
                _close(lse[b, hq], s, tol=1e-11, what=f"single-token score at {q_pos}")


def pin_append_rounding(library):
    """bf16 storage: the new key is the rotation rounded once to bf16."""
    p = ragged_problem(46, B=3, Hkv=2, G=2, d=64, ncap=5, rk=16, rv=16, wcap=4, theta=500000.0,
                       q_pos=40000)
    bits = {}
    for name in ("q", "U_K", "U_V", "C_K", "C_V", "K_raw", "V_raw", "k_new", "v_new"):
        bits[name] = (p[name].astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    pb = dict(p)
    pb.update(bits)
    _, _, k_app = run_ragged(pb, library)
    rot = rope_complex(oracle.bf16_to_f64(bits["k_new"]), p["q_pos"][:, None], p["theta"])
    assert np.array_equal(k_app, bf16_round(rot)), "new key not rounded once to bf16"


def pin_append_rounding_fp32(library):
    """fp32 storage: the new key is the rotation rounded once to fp32 (IEEE
    round to nearest even, as numpy's float64 -> float32 conversion does),
    not kept in double and not rounded twice through bf16."""
    p = ragged_problem(47, B=3, Hkv=2, G=2, d=64, ncap=5, rk=16, rv=16, wcap=4, theta=500000.0,
                       q_pos=40000)
    pf = dict(p)
    for name in ("q", "U_K", "U_V", "C_K", "C_V", "K_raw", "V_raw", "k_new", "v_new"):
        pf[name] = p[name].astype(np.float32)
    _, _, k_app = run_ragged(pf, library)
    rot = rope_complex(pf["k_new"].astype(np.float64), p["q_pos"][:, None], p["theta"])
    want = rot.astype(np.float32).astype(np.float64)
    assert np.array_equal(np.asarray(k_app, dtype=np.float64), want), \
        "new key not rounded once to fp32"
    assert not np.array_equal(want, rot), "fixture too coarse: rounding never changes a value"


# ---------------------------------------------------------------------------
# The reconstruction variant that keeps beacon-key rotation (oracle.decode
# with beacon_pos): rebuilt beacon keys are rotated at their positions.


def beacon_rope_reference(p, beacon_pos):
    """Independent statement: rebuild C_K U_K^T and C_V U_V^T, rotate the
    rebuilt keys at their positions (complex multiplication), append the raw
    rows, and run torch's SDPA with the rotated query."""
    G = p["q"].shape[1] // p["num_kv_heads"]
    q_rot = rope_complex(p["q"], p["q_pos"][:, None], p["theta"])
    kb = np.einsum("bhjr,hdr->bhjd", p["C_K"], p["U_K"])
    kb = rope_complex(kb, np.asarray(beacon_pos)[None, None, :], p["theta"])
    vb = np.einsum("bhjr,hdr->bhjd", p["C_V"], p["U_V"])
    K = np.concatenate([kb, p["K_raw"]], axis=2)
    V = np.concatenate([vb, p["V_raw"]], axis=2)
    return sdpa_reference(q_rot, K, V, p["scale"], G)


def pin_beacon_rope_reference(library):
    for seed, shape in ((60, dict(B=2, Hkv=2, G=4, d=16, nb=17, rk=4, rv=8, w=3)),
                        (61, dict(B=1, Hkv=2, G=5, d=128, nb=33, rk=32, rv=48, w=9, theta=500000.0,
                                  q_pos=131071))):
        p = random_problem(seed, **shape)
        ratio = 16
        bpos = ((np.arange(shape["nb"]) + 1) * ratio - 1).astype(np.int32)
        out, lse = run_oracle(p, library, beacon_pos=bpos)
        ref_out, ref_lse = beacon_rope_reference(p, bpos)
        _close(out, ref_out, tol=1e-10, what=f"beacon-rope out {shape}")
        _close(lse, ref_lse, tol=1e-10, what=f"beacon-rope lse {shape}")


def pin_beacon_rope_relative(library):
    """Beacons at the query position turn with the query, so (no raw rows)
    the scores are those of the unrotated query against the unrotated keys:
    the latent path with the query at position 0.  Shifting the query, the
    beacons and the raw keys together leaves the output unchanged; moving
    only the beacons changes it."""
    pb = random_problem(63, B=2, Hkv=1, G=4, d=32, nb=9, rk=8, rv=8, w=0, q_pos=777)
    out, lse = run_oracle(pb, library, beacon_pos=np.full(9, 777, dtype=np.int32))
    lat, lat_lse = run_oracle(pb, library, q_pos=np.zeros(2, dtype=np.int32))
    _close(out, lat, tol=1e-11, what="beacons at the query position")
    _close(lse, lat_lse, tol=1e-11, what="beacons at the query position, lse")
    p = random_problem(62, B=2, Hkv=1, G=4, d=32, nb=9, rk=8, rv=8, w=5, q_pos=777)
    bpos = (np.arange(9) * 50 + 3).astype(np.int32)
    out0, _ = run_oracle(p, library, beacon_pos=bpos)
    shift = 100000
    qp = p["q_pos"] + shift
    raw_pos = qp[:, None] - 5 + 1 + np.arange(5)[None, :]
    k = rope_complex(p["K_pre"], raw_pos[:, None, :], p["theta"])
    out1, _ = run_oracle(p, library, q_pos=qp.astype(np.int32), K_raw=k,
                         beacon_pos=(bpos + shift).astype(np.int32))
    _close(out1, out0, tol=1e-9, what="beacon-rope shift")
    out2, _ = run_oracle(p, library, beacon_pos=(bpos + 7).astype(np.int32))
    assert np.max(np.abs(out2 - out0)) > 1e-6, "beacon positions have no effect"


# ---------------------------------------------------------------------------
# Chunks of several query tokens per sequence (oracle.decode_chunk).


def chunk_problem(seed, *, Q=3, room=True, **shape):
    """A ragged problem with Q query tokens per sequence and Q new tokens;
    room: every sequence's window has space for the whole chunk."""
    p = ragged_problem(seed, append=False, **shape)
    rng = np.random.default_rng(seed + 2000)
    B, Hq, d = p["q"].shape
    Hkv, wcap = p["num_kv_heads"], p["K_raw"].shape[2]
    p["q"] = rng.standard_normal((B, Q, Hq, d))
    p["k_new"] = rng.standard_normal((B, Q, Hkv, d))
    p["v_new"] = rng.standard_normal((B, Q, Hkv, d))
    if room:
        p["raw_len"] = rng.integers(0, wcap - Q + 1, size=B).astype(np.int32)
    return p


def run_chunk(p, library, **over):
    args = dict(p)
    args.update(over)
    ncap = args["C_K"].shape[2]
    wcap = args["K_raw"].shape[2]
    return oracle.decode_chunk(
        args["q"], args["q_pos"], args["U_K"], args["U_V"],
        args["C_K"] if ncap else None, args["C_V"] if ncap else None,
        args["K_raw"] if wcap else None, args["V_raw"] if wcap else None,
        num_kv_heads=args["num_kv_heads"], scale=args["scale"], rope_theta=args["theta"],
        num_beacons=args.get("num_beacons"), raw_len=args.get("raw_len"),
        k_new=args.get("k_new"), v_new=args.get("v_new"), library=library)


def chunk_reference(p, b, t):
    """Token t of sequence b: its live beacon rows rebuilt to full keys and
    values, its live raw rows, and the chunk's tokens 0..t (token u's key
    rotated at q_pos[b] + u); ordinary attention of the query rotated at
    q_pos[b] + t.  Returns (out [H_q, d], lse [H_q])."""
    Hkv = p["num_kv_heads"]
    G = p["q"].shape[2] // Hkv
    nbc = int(np.clip(p["num_beacons"][b], 0, p["C_K"].shape[2]))
    wc = int(np.clip(p["raw_len"][b], 0, p["K_raw"].shape[2]))
    pos = int(p["q_pos"][b])
    K = [np.einsum("hjr,hdr->hjd", p["C_K"][b, :, :nbc], p["U_K"]), p["K_raw"][b, :, :wc]]
    V = [np.einsum("hjr,hdr->hjd", p["C_V"][b, :, :nbc], p["U_V"]), p["V_raw"][b, :, :wc]]
    for u in range(t + 1):
        K.append(rope_complex(p["k_new"][b, u], np.full(Hkv, pos + u), p["theta"])[:, None, :])
        V.append(p["v_new"][b, u][:, None, :])
    K = np.concatenate(K, axis=1)[None]
    V = np.concatenate(V, axis=1)[None]
    q_rot = rope_complex(p["q"][b:b + 1, t], np.array([[pos + t]]), p["theta"])
    out, lse = sdpa_reference(q_rot, K, V, p["scale"], G)
    return out[0], lse[0]


def pin_chunk_reference(library):
    """Each token of a chunk against plain attention over the cache rows and
    the chunk's tokens up to it; full windows included (the chunk is
    attended whether or not it can be stored)."""
    for seed, shape in ((60, dict(B=4, Hkv=2, G=2, d=16, ncap=6, rk=4, rv=6, wcap=7)),
                        (61, dict(B=2, Hkv=1, G=3, d=128, ncap=20, rk=32, rv=16, wcap=4,
                                  theta=500000.0, q_pos=131060))):
        p = chunk_problem(seed, Q=3, room=False, **shape)
        p["raw_len"][0] = shape["wcap"]
        p["num_beacons"][1] = 0
        out, lse, _ = run_chunk(p, library)
        for b in range(shape["B"]):
            for t in range(3):
                ref_out, ref_lse = chunk_reference(p, b, t)
                _close(out[b, t], ref_out, what=f"chunk out, seq {b} token {t}")
                _close(lse[b, t], ref_lse, what=f"chunk lse, seq {b} token {t}")


def pin_chunk_single_token(library):
    """A chunk of one token is the ragged decode step."""
    p = chunk_problem(62, Q=1, room=False, B=5, Hkv=2, G=2, d=16, ncap=9, rk=4, rv=6, wcap=7)
    out, lse, k_app = run_chunk(p, library)
    r_out, r_lse, r_k = run_ragged(p, library, q=p["q"][:, 0], k_new=p["k_new"][:, 0],
                                   v_new=p["v_new"][:, 0])
    _close(out[:, 0], r_out, tol=1e-13, what="chunk of one: out")
    _close(lse[:, 0], r_lse, tol=1e-13, what="chunk of one: lse")
    _close(k_app[:, 0], r_k, tol=1e-14, what="chunk of one: stored key")


def pin_chunk_sequential(library):
    """A chunk equals its tokens decoded one after another, each step
    appending its token to the raw window before the next (the window has
    room for all of them)."""
    for seed, shape in ((63, dict(B=4, Hkv=2, G=2, d=16, ncap=6, rk=4, rv=6, wcap=9)),
                        (64, dict(B=3, Hkv=2, G=1, d=32, ncap=0, rk=4, rv=4, wcap=8))):
        Q = 4
        p = chunk_problem(seed, Q=Q, **shape)
        out, lse, k_app = run_chunk(p, library)
        K, V = p["K_raw"].copy(), p["V_raw"].copy()
        for t in range(Q):
            o, l_, k = run_ragged(p, library, q=p["q"][:, t], q_pos=(p["q_pos"] + t).astype(np.int32),
                                  K_raw=K, V_raw=V, raw_len=(p["raw_len"] + t).astype(np.int32),
                                  k_new=p["k_new"][:, t], v_new=p["v_new"][:, t])
            _close(out[:, t], o, tol=1e-12, what=f"sequential out, token {t}")
            _close(lse[:, t], l_, tol=1e-12, what=f"sequential lse, token {t}")
            _close(k_app[:, t], k, tol=1e-14, what=f"sequential stored key, token {t}")
            for b in range(shape["B"]):
                K[b, :, p["raw_len"][b] + t] = k[b]
                V[b, :, p["raw_len"][b] + t] = p["v_new"][b, t]


def pin_chunk_causal(library):
    """Token t sees the chunk's tokens up to t only: changing later tokens
    leaves its output untouched, changing token t does not."""
    p = chunk_problem(65, Q=4, B=3, Hkv=2, G=2, d=16, ncap=5, rk=4, rv=4, wcap=9)
    out, lse, _ = run_chunk(p, library)
    for t in range(3):
        k2, v2 = p["k_new"].copy(), p["v_new"].copy()
        k2[:, t + 1:] += 3.0
        v2[:, t + 1:] -= 2.0
        o2, l2, _ = run_chunk(p, library, k_new=k2, v_new=v2)
        assert np.array_equal(o2[:, :t + 1], out[:, :t + 1]), f"token {t} sees later tokens"
        assert np.array_equal(l2[:, :t + 1], lse[:, :t + 1])
        assert np.max(np.abs(o2[:, t + 1:] - out[:, t + 1:])) > 1e-6, "later tokens ignored"


def pin_chunk_without_new_tokens(library):
    """Without new tokens each query of the chunk attends over the cache only,
    at its own position."""
    p = chunk_problem(66, Q=3, room=False, B=3, Hkv=2, G=2, d=16, ncap=6, rk=4, rv=4, wcap=5)
    out, lse, k_app = run_chunk(p, library, k_new=None, v_new=None)
    assert np.all(np.isnan(k_app))
    for t in range(3):
        o, l_, _ = run_ragged(p, library, q=p["q"][:, t], q_pos=(p["q_pos"] + t).astype(np.int32),
                              k_new=None, v_new=None)
        _close(out[:, t], o, tol=1e-13, what=f"no new tokens, token {t}")
        _close(lse[:, t], l_, tol=1e-13, what=f"no new tokens lse, token {t}")


def pin_chunk_rounding(library):
    """bf16 storage: each new key is its rotation at its own position, rounded
    once to bf16."""
    p = chunk_problem(67, Q=3, room=False, B=2, Hkv=2, G=2, d=64, ncap=5, rk=16, rv=16, wcap=4,
                      theta=500000.0, q_pos=70000)
    bits = {}
    for name in ("q", "U_K", "U_V", "C_K", "C_V", "K_raw", "V_raw", "k_new", "v_new"):
        bits[name] = (p[name].astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    pb = dict(p)
    pb.update(bits)
    _, _, k_app = run_chunk(pb, library)
    pos = p["q_pos"][:, None, None] + np.arange(3)[None, :, None]
    rot = rope_complex(oracle.bf16_to_f64(bits["k_new"]), pos, p["theta"])
    assert np.array_equal(k_app, bf16_round(rot)), "chunk keys not rounded once to bf16"


# ---------------------------------------------------------------------------
# The ALiBi variant (oracle.decode_alibi): no rotation, a linear distance
# bias on every score.


def run_alibi(p, library, **over):
    args = dict(p)
    args.update(over)
    nb = args["C_K"].shape[2]
    return oracle.decode_alibi(
        args["q"], args["q_pos"], args["U_K"], args["U_V"], args["C_K"] if nb else None,
        args["C_V"] if nb else None, args["K_raw"], args["V_raw"],
        beacon_pos=args["beacon_pos"], slopes=args["slopes"],
        num_kv_heads=args["num_kv_heads"], scale=args["scale"], library=library)


def alibi_problem(seed, *, ratio=4, q_pos=None, **shape):
    p = random_problem(seed, q_pos=q_pos, **shape)
    nb = p["C_K"].shape[2]
    p["beacon_pos"] = ((np.arange(nb) + 1) * ratio - 1).astype(np.int32)
    rng = np.random.default_rng(seed + 3000)
    p["slopes"] = rng.uniform(0.01, 0.5, size=p["q"].shape[1])
    return p


def alibi_reference(p):
    """Plain attention over the rebuilt beacon rows and the raw rows, no
    rotation, scores scale * q.k - slope * (q_pos - k_pos)."""
    q = p["q"]
    B, Hq, d = q.shape
    Hkv = p["num_kv_heads"]
    G = Hq // Hkv
    w = p["K_raw"].shape[2]
    kb = np.einsum("bhjr,hdr->bhjd", p["C_K"], p["U_K"])
    vb = np.einsum("bhjr,hdr->bhjd", p["C_V"], p["U_V"])
    K = np.concatenate([kb, p["K_raw"]], axis=2)
    V = np.concatenate([vb, p["V_raw"]], axis=2)
    out = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    for b in range(B):
        qp = int(p["q_pos"][b])
        kpos = np.concatenate([p["beacon_pos"], qp - w + 1 + np.arange(w)]).astype(np.float64)
        for hq in range(Hq):
            h = hq // G
            s = p["scale"] * (K[b, h] @ q[b, hq]) - p["slopes"][hq] * (qp - kpos)
            m = s.max()
            e = np.exp(s - m)
            out[b, hq] = e @ V[b, h] / e.sum()
            lse[b, hq] = m + np.log(e.sum())
    return out, lse


def pin_alibi_reference(library):
    for seed, shape in ((70, dict(B=2, Hkv=2, G=2, d=16, nb=6, rk=4, rv=6, w=5)),
                        (71, dict(B=1, Hkv=1, G=4, d=128, nb=40, rk=32, rv=16, w=9,
                                  q_pos=131071))):
        p = alibi_problem(seed, **shape)
        out, lse = run_alibi(p, library)
        ref, ref_lse = alibi_reference(p)
        _close(out, ref, what=f"alibi out {shape}")
        _close(lse, ref_lse, what=f"alibi lse {shape}")


def pin_alibi_zero_slopes(library):
    """Without bias, an ALiBi backbone's attention is RoPE attention at
    position 0 (every rotation the identity)."""
    p = alibi_problem(72, B=2, Hkv=2, G=3, d=32, nb=7, rk=8, rv=8, w=4, q_pos=5000)
    out, lse = run_alibi(p, library, slopes=np.zeros(6))
    ref, ref_lse = run_oracle(p, library, q_pos=np.zeros(2, dtype=np.int32))
    _close(out, ref, tol=1e-13, what="alibi without bias")
    _close(lse, ref_lse, tol=1e-13, what="alibi without bias lse")


def pin_alibi_translation(library):
    """Only distances count: moving the query and the beacons by the same
    offset (raw rows move with the query) changes nothing."""
    p = alibi_problem(73, B=2, Hkv=1, G=2, d=16, nb=6, rk=4, rv=4, w=5, q_pos=30)
    out, lse = run_alibi(p, library)
    out2, lse2 = run_alibi(p, library, q_pos=(p["q_pos"] + 99991).astype(np.int32),
                           beacon_pos=(p["beacon_pos"] + 99991).astype(np.int32))
    _close(out2, out, tol=1e-12, what="alibi translation")
    _close(lse2, lse - 0.0, tol=1e-9, what="alibi translation lse")
    out3, _ = run_alibi(p, library, beacon_pos=(p["beacon_pos"] + 3).astype(np.int32))
    assert np.max(np.abs(out3 - out)) > 1e-6, "beacon positions have no effect"


def pin_alibi_two_rows(library):
    """One beacon and one raw row: a two-way softmax in closed form."""
    p = alibi_problem(74, B=1, Hkv=1, G=1, d=8, nb=1, rk=4, rv=4, w=1, q_pos=50)
    p["beacon_pos"] = np.array([20], dtype=np.int32)
    out, lse = run_alibi(p, library)
    q = p["q"][0, 0]
    kb = p["U_K"][0] @ p["C_K"][0, 0, 0]
    vb = p["U_V"][0] @ p["C_V"][0, 0, 0]
    m = p["slopes"][0]
    s0 = p["scale"] * q @ kb - m * 30.0          # beacon at distance 30
    s1 = p["scale"] * q @ p["K_raw"][0, 0, 0]    # the raw row sits at the query's position
    a0 = 1.0 / (1.0 + np.exp(s1 - s0))
    _close(out[0, 0], a0 * vb + (1.0 - a0) * p["V_raw"][0, 0, 0], what="two-row alibi")
    _close(lse[0, 0], np.logaddexp(s0, s1), what="two-row alibi lse")


def pin_alibi_steep(library):
    """A steep slope leaves only the nearest row: the raw row at the query's
    position."""
    p = alibi_problem(75, B=2, Hkv=1, G=2, d=16, nb=5, rk=4, rv=4, w=4, q_pos=100)
    out, _ = run_alibi(p, library, slopes=np.full(2, 200.0))
    for b in range(2):
        for hq in range(2):
            _close(out[b, hq], p["V_raw"][b, 0, -1], tol=1e-12, what="steep alibi")



# ---------------------------------------------------------------------------
# The ALiBi variant of a serving step (oracle.decode_chunk_alibi): ragged
# lengths, new tokens and several query tokens per sequence.  Positions:
# query token t at q_pos + t, beacon j at beacon_pos[j], new token u at
# q_pos + u, live raw row i at q_pos - w + i with new tokens (they follow the
# raw rows) and q_pos - w + 1 + i without.


def alibi_step_problem(seed, *, Q=1, append=True, **shape):
    p = ragged_problem(seed, append=False, **shape)
    nb = p["C_K"].shape[2]
    rng = np.random.default_rng(seed + 4000)
    B, Hkv, d = p["q"].shape[0], p["num_kv_heads"], p["q"].shape[2]
    Hq = p["q"].shape[1]
    p["q"] = rng.standard_normal((B, Q, Hq, d))
    p["q_pos"] = rng.integers(50, 200, size=B).astype(np.int32)
    p["beacon_pos"] = ((np.arange(nb) + 1) * 4 - 1).astype(np.int32)
    p["slopes"] = rng.uniform(0.01, 0.5, size=Hq)
    if append:
        p["k_new"] = rng.standard_normal((B, Q, Hkv, d))
        p["v_new"] = rng.standard_normal((B, Q, Hkv, d))
    return p


def run_alibi_step(p, library, **over):
    args = dict(p)
    args.update(over)
    ncap = args["C_K"].shape[2]
    wcap = args["K_raw"].shape[2]
    return oracle.decode_chunk_alibi(
        args["q"], args["q_pos"], args["U_K"], args["U_V"],
        args["C_K"] if ncap else None, args["C_V"] if ncap else None,
        args["K_raw"] if wcap else None, args["V_raw"] if wcap else None,
        beacon_pos=args["beacon_pos"], slopes=args["slopes"], num_kv_heads=args["num_kv_heads"],
        scale=args["scale"], num_beacons=args.get("num_beacons"), raw_len=args.get("raw_len"),
        k_new=args.get("k_new"), v_new=args.get("v_new"), library=library)


def alibi_step_reference(p):
    """Each sequence and query token alone: the live beacon rows rebuilt to
    full width, the live raw rows and the new tokens up to the query, listed
    with their positions; plain attention with the bias."""
    q = p["q"]
    B, Q, Hq, d = q.shape
    Hkv = p["num_kv_heads"]
    G = Hq // Hkv
    out = np.zeros((B, Q, Hq, d))
    lse = np.zeros((B, Q, Hq))
    app = p.get("k_new") is not None
    for b in range(B):
        nbc = int(np.clip(p["num_beacons"][b], 0, p["C_K"].shape[2]))
        wc = int(np.clip(p["raw_len"][b], 0, p["K_raw"].shape[2]))
        qp = int(p["q_pos"][b])
        for t in range(Q):
            for hq in range(Hq):
                h = hq // G
                keys = [p["C_K"][b, h, j] @ p["U_K"][h].T for j in range(nbc)]
                vals = [p["C_V"][b, h, j] @ p["U_V"][h].T for j in range(nbc)]
                pos = [int(p["beacon_pos"][j]) for j in range(nbc)]
                first_raw = qp - wc if app else qp - wc + 1
                keys += [p["K_raw"][b, h, i] for i in range(wc)]
                vals += [p["V_raw"][b, h, i] for i in range(wc)]
                pos += [first_raw + i for i in range(wc)]
                if app:
                    keys += [p["k_new"][b, u, h] for u in range(t + 1)]
                    vals += [p["v_new"][b, u, h] for u in range(t + 1)]
                    pos += [qp + u for u in range(t + 1)]
                if not keys:
                    lse[b, t, hq] = -np.inf
                    continue
                K, V = np.array(keys), np.array(vals)
                sc = p["scale"] * (K @ q[b, t, hq]) - p["slopes"][hq] * (qp + t - np.array(pos, float))
                m = sc.max()
                e = np.exp(sc - m)
                out[b, t, hq] = e @ V / e.sum()
                lse[b, t, hq] = m + np.log(e.sum())
    return out, lse


def pin_alibi_step_reference(library):
    """Ragged lengths (clamped), new tokens, several query tokens: each
    sequence against plain attention over its listed rows and positions."""
    for seed, Q, app, shape in ((80, 1, True, dict(B=4, Hkv=2, G=2, d=16, ncap=9, rk=4, rv=6, wcap=7)),
                                (81, 3, True, dict(B=3, Hkv=1, G=4, d=32, ncap=6, rk=8, rv=4, wcap=5)),
                                (82, 2, False, dict(B=3, Hkv=2, G=1, d=16, ncap=5, rk=4, rv=4, wcap=6)),
                                (83, 2, True, dict(B=2, Hkv=1, G=2, d=16, ncap=0, rk=4, rv=4, wcap=4))):
        p = alibi_step_problem(seed, Q=Q, append=app, **shape)
        if shape["B"] > 2:
            p["num_beacons"][1] = 0
            p["raw_len"][1] = 0
            p["num_beacons"][2] = shape["ncap"] + 3  # clamped
            p["raw_len"][2] = -1
        out, lse, k_app = run_alibi_step(p, library)
        ref, ref_lse = alibi_step_reference(p)
        _close(out, ref, what=f"alibi step out Q={Q} app={app}")
        fin = np.isfinite(ref_lse)
        assert np.array_equal(fin, np.isfinite(lse)), "alibi step: empty rows"
        _close(lse[fin], ref_lse[fin], what=f"alibi step lse Q={Q}")
        if app:
            _close(k_app, p["k_new"], tol=0.0, what="alibi new keys are stored as given")


def pin_alibi_step_is_uniform_alibi(library):
    """Full lengths, no new tokens, one query token: exactly the uniform
    ALiBi variant (whose raw window also ends at the query)."""
    p = alibi_step_problem(84, Q=1, append=False, B=2, Hkv=2, G=3, d=16, ncap=7, rk=4, rv=6, wcap=5)
    p["num_beacons"][:] = 7
    p["raw_len"][:] = 5
    out, lse, _ = run_alibi_step(p, library)
    ref, ref_lse = oracle.decode_alibi(p["q"][:, 0], p["q_pos"], p["U_K"], p["U_V"], p["C_K"],
                                       p["C_V"], p["K_raw"], p["V_raw"],
                                       beacon_pos=p["beacon_pos"], slopes=p["slopes"],
                                       num_kv_heads=2, scale=p["scale"], library=library)
    _close(out[:, 0], ref, tol=1e-14, what="alibi step vs uniform alibi")
    _close(lse[:, 0], ref_lse, tol=1e-14, what="alibi step vs uniform alibi lse")


def pin_alibi_step_sequential(library):
    """A chunk of Q tokens equals Q single-token steps, each appending its
    token (raw_len + 1) at the next position (q_pos + 1): the positions of
    the chunk's rows and tokens agree with those of the steps."""
    Q = 3
    p = alibi_step_problem(85, Q=Q, B=2, Hkv=1, G=2, d=16, ncap=5, rk=4, rv=4, wcap=9)
    p["raw_len"][:] = [3, 5]
    out, lse, _ = run_alibi_step(p, library)
    K, V = p["K_raw"].copy(), p["V_raw"].copy()
    for t in range(Q):
        for b in range(2):
            w = int(p["raw_len"][b]) + t
            if t:
                K[b, :, w - 1] = p["k_new"][b, t - 1]
                V[b, :, w - 1] = p["v_new"][b, t - 1]
        o1, l1, _ = run_alibi_step(p, library, q=p["q"][:, t:t + 1], q_pos=p["q_pos"] + t,
                                   raw_len=p["raw_len"] + t, K_raw=K, V_raw=V,
                                   k_new=p["k_new"][:, t:t + 1], v_new=p["v_new"][:, t:t + 1])
        _close(out[:, t], o1[:, 0], what=f"alibi chunk token {t} vs a step")
        _close(lse[:, t], l1[:, 0], what=f"alibi chunk token {t} vs a step lse")


def pin_alibi_step_causal_and_translation(library):
    """Later tokens do not reach earlier queries; moving every position
    (queries and beacons) by one offset changes nothing."""
    p = alibi_step_problem(86, Q=3, B=2, Hkv=2, G=2, d=16, ncap=6, rk=4, rv=4, wcap=6)
    out, lse, _ = run_alibi_step(p, library)
    kn = p["k_new"].copy()
    kn[:, 2] += 5.0
    out2, _, _ = run_alibi_step(p, library, k_new=kn)
    assert np.array_equal(out[:, :2], out2[:, :2]), "a later token reached an earlier query"
    assert not np.allclose(out[:, 2], out2[:, 2]), "the last token's own key is unused"
    out3, lse3, _ = run_alibi_step(p, library, q_pos=p["q_pos"] + 1000,
                                   beacon_pos=p["beacon_pos"] + 1000)
    _close(out3, out, tol=1e-12, what="alibi step translation")
    _close(lse3, lse, tol=1e-12, what="alibi step translation lse")


def pin_alibi_step_token_only(library):
    """A sequence holding only its new token: output its value, lse the plain
    scaled score (zero distance to itself), at any position."""
    for qp in (0, 99, 131071):
        p = alibi_step_problem(87, Q=1, B=2, Hkv=2, G=2, d=16, ncap=4, rk=4, rv=4, wcap=3)
        p["num_beacons"][:] = 0
        p["raw_len"][:] = 0
        p["q_pos"][:] = qp
        out, lse, _ = run_alibi_step(p, library)
        for b in range(2):
            for hq in range(4):
                h = hq // 2
                _close(out[b, 0, hq], p["v_new"][b, 0, h], tol=1e-14, what="token-only out")
                s = p["scale"] * float(p["q"][b, 0, hq] @ p["k_new"][b, 0, h])
                _close(lse[b, 0, hq], s, tol=1e-12, what=f"token-only lse at {qp}")


ALL_PINS = [
    pin_reconstruct_identity,
    pin_raw_only_rope_gqa,
    pin_beacon_keys_unrotated,
    pin_relative_position,
    pin_position_zero,
    pin_constant_values,
    pin_rebasing,
    pin_permutations,
    pin_closed_forms,
    pin_ragged_lengths,
    pin_append_token,
    pin_append_self_score,
    pin_append_rounding,
    pin_append_rounding_fp32,
    pin_beacon_rope_reference,
    pin_beacon_rope_relative,
    pin_chunk_reference,
    pin_chunk_single_token,
    pin_chunk_sequential,
    pin_chunk_causal,
    pin_chunk_without_new_tokens,
    pin_chunk_rounding,
    pin_alibi_reference,
    pin_alibi_zero_slopes,
    pin_alibi_translation,
    pin_alibi_two_rows,
    pin_alibi_steep,
    pin_alibi_step_reference,
    pin_alibi_step_is_uniform_alibi,
    pin_alibi_step_sequential,
    pin_alibi_step_causal_and_translation,
    pin_alibi_step_token_only,
]
