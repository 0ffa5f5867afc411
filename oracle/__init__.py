"""fp64 CPU oracle for SlimKV latent decode attention -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The HIP library never does, and this package
never imports the library: the two share no code.

``decode`` runs the plain C implementation in ``slimkv_oracle.c`` (double
precision throughout, OpenMP over (batch, kv head) units); ``decode_ragged``
the same with per-sequence lengths and the decode step's new token;
``decode_chunk`` a chunk of several query tokens per sequence; ``decode_alibi``
and ``decode_chunk_alibi`` the ALiBi variant (no rotation, a distance bias).  Its definition
follows page "Can SlimKV compress KV cache jointly across tokens and
features", section "Latent-space attention removes the rebuild step": the
rotated query is projected into each KV head's beacon latent space, scored
against rotation-free latent beacon keys and rotated raw-token keys under one
softmax, and the latent value sum is lifted once by U_V.
"""

from __future__ import annotations

import ctypes
import os
import pathlib
import subprocess

import numpy as np

HERE = pathlib.Path(__file__).resolve().parent
SOURCE = HERE / "slimkv_oracle.c"
LIBRARY = HERE / "libslimkv_oracle.so"

_DTYPE = {np.dtype(np.float64): 0, np.dtype(np.float32): 1, np.dtype(np.uint16): 2}


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("num_beacons", ctypes.c_int32),
        ("rank_k", ctypes.c_int32),
        ("rank_v", ctypes.c_int32),
        ("raw_window", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("rope_theta", ctypes.c_double),
        ("dtype", ctypes.c_int32),
    ]


def build(source: pathlib.Path = SOURCE, target: pathlib.Path = LIBRARY) -> pathlib.Path:
    """Compile the C oracle with gcc (always rebuilds)."""
    tmp = f"{target}.{os.getpid()}.tmp"  # concurrent builds each write their own file
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           str(source), "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, target)
    return target


_lib_cache: dict = {}


def load(path=LIBRARY) -> ctypes.CDLL:
    path = pathlib.Path(path)
    key = str(path)
    if key not in _lib_cache:
        if not path.exists():
            build(target=path)
        lib = ctypes.CDLL(key)
        lib.slimkv_oracle_decode.restype = ctypes.c_int
        lib.slimkv_oracle_decode.argtypes = [ctypes.POINTER(_Problem)] + [ctypes.c_void_p] * 8 + [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        if hasattr(lib, "slimkv_oracle_decode_beacon_rope"):
            lib.slimkv_oracle_decode_beacon_rope.restype = ctypes.c_int
            lib.slimkv_oracle_decode_beacon_rope.argtypes = [ctypes.POINTER(_Problem)] + [
                ctypes.c_void_p] * 9 + [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_int]
        if hasattr(lib, "slimkv_oracle_decode_ragged"):
            lib.slimkv_oracle_decode_ragged.restype = ctypes.c_int
            lib.slimkv_oracle_decode_ragged.argtypes = [ctypes.POINTER(_Problem)] + [
                ctypes.c_void_p] * 12 + [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        if hasattr(lib, "slimkv_oracle_decode_chunk"):
            lib.slimkv_oracle_decode_chunk.restype = ctypes.c_int
            lib.slimkv_oracle_decode_chunk.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int] + [
                ctypes.c_void_p] * 12 + [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        if hasattr(lib, "slimkv_oracle_decode_alibi"):
            lib.slimkv_oracle_decode_alibi.restype = ctypes.c_int
            lib.slimkv_oracle_decode_alibi.argtypes = [ctypes.POINTER(_Problem)] + [
                ctypes.c_void_p] * 10 + [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_int]
        if hasattr(lib, "slimkv_oracle_decode_chunk_alibi"):
            lib.slimkv_oracle_decode_chunk_alibi.restype = ctypes.c_int
            lib.slimkv_oracle_decode_chunk_alibi.argtypes = [
                ctypes.POINTER(_Problem), ctypes.c_int] + [ctypes.c_void_p] * 14 + [
                ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                ctypes.c_void_p, ctypes.c_int]
        lib.slimkv_oracle_max_threads.restype = ctypes.c_int
        _lib_cache[key] = lib
    return _lib_cache[key]


def max_threads() -> int:
    return int(load().slimkv_oracle_max_threads())


def _arr(x, dtype):
    if x is None:
        return None
    a = np.ascontiguousarray(x)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def decode(q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw, *, num_kv_heads: int, scale: float,
           rope_theta: float, units=None, threads: int = 0, library: pathlib.Path = LIBRARY,
           beacon_pos=None):
    """fp64 latent decode attention.

    Arrays are numpy, row-major, all in one storage dtype (float64, float32,
    or uint16 holding bf16 bits):
        q [B, H_q, d], q_pos [B] int32, U_K [H_kv, d, r_K], U_V [H_kv, d, r_V],
        C_K [B, H_kv, N_b, r_K], C_V [B, H_kv, N_b, r_V],
        K_raw [B, H_kv, W, d] (already rotated), V_raw [B, H_kv, W, d].
    C_K/C_V (or K_raw/V_raw) may be None when N_b (or W) is 0.
    ``units`` is an optional list of (b, kv_head) pairs to compute; other
    rows of the result stay NaN.  Returns (out [B, H_q, d], lse [B, H_q]) in
    float64; lse is in natural-log units of the scaled scores.
    ``beacon_pos`` ([N_b] int32) selects the reconstruction variant that keeps
    beacon-key rotation: beacon j's key is rebuilt as U_K C_K[j] and rotated
    at beacon_pos[j] before it is scored.
    """
    q = np.ascontiguousarray(q)
    dt = q.dtype
    if dt not in _DTYPE:
        raise TypeError(f"unsupported storage dtype {dt}")
    B, Hq, d = q.shape
    q_pos = _arr(q_pos, np.dtype(np.int32))
    nb = 0 if C_K is None else int(np.shape(C_K)[2])
    w = 0 if K_raw is None else int(np.shape(K_raw)[2])
    rk = int(np.shape(U_K)[2]) if U_K is not None else 0
    rv = int(np.shape(U_V)[2]) if U_V is not None else 0
    U_K, U_V, C_K, C_V, K_raw, V_raw = (_arr(x, dt) for x in (U_K, U_V, C_K, C_V, K_raw, V_raw))
    prob = _Problem(B, Hq, num_kv_heads, d, nb, rk, rv, w, float(scale), float(rope_theta),
                    _DTYPE[dt])
    out = np.full((B, Hq, d), np.nan, dtype=np.float64)
    lse = np.full((B, Hq), np.nan, dtype=np.float64)
    if units is None:
        unit_arr, n_units = None, 0
    else:
        unit_arr = np.ascontiguousarray(np.asarray(units, dtype=np.int32).reshape(-1, 2))
        n_units = unit_arr.shape[0]

    def ptr(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    if beacon_pos is None:
        rc = load(library).slimkv_oracle_decode(
            ctypes.byref(prob), ptr(q), ptr(q_pos), ptr(U_K), ptr(U_V), ptr(C_K), ptr(C_V),
            ptr(K_raw), ptr(V_raw), ptr(unit_arr), n_units, ptr(out), ptr(lse), int(threads))
    else:
        bp = _arr(beacon_pos, np.dtype(np.int32))
        rc = load(library).slimkv_oracle_decode_beacon_rope(
            ctypes.byref(prob), ptr(q), ptr(q_pos), ptr(U_K), ptr(U_V), ptr(C_K), ptr(C_V),
            ptr(K_raw), ptr(V_raw), ptr(bp), ptr(unit_arr), n_units, ptr(out), ptr(lse),
            int(threads))
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    return out, lse


def decode_ragged(q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw, *, num_kv_heads: int, scale: float,
                  rope_theta: float, num_beacons=None, raw_len=None, k_new=None, v_new=None,
                  units=None, threads: int = 0, library: pathlib.Path = LIBRARY):
    """fp64 decode attention over a ragged batch, with the step's new token.

    The cache arrays are as for ``decode`` but sized to capacities: C_K
    [B, H_kv, N_cap, r_K] etc., K_raw [B, H_kv, W_cap, d].  ``num_beacons``
    and ``raw_len`` ([B] int32, None = the capacity) give each sequence's
    live rows (clamped to [0, capacity]).  ``k_new``, ``v_new`` ([B, H_kv, d],
    storage dtype, both or neither) are the new token's key before rotation
    and its value: the key is rotated at q_pos[b], rounded to the storage
    precision and attended as one more raw row.  Returns (out, lse, k_app):
    k_app [B, H_kv, d] float64 holds the rounded rotated new keys (NaN
    without a new token).  A sequence without rows gets out 0, lse -inf.
    """
    q = np.ascontiguousarray(q)
    dt = q.dtype
    if dt not in _DTYPE:
        raise TypeError(f"unsupported storage dtype {dt}")
    B, Hq, d = q.shape
    q_pos = _arr(q_pos, np.dtype(np.int32))
    ncap = 0 if C_K is None else int(np.shape(C_K)[2])
    wcap = 0 if K_raw is None else int(np.shape(K_raw)[2])
    rk = int(np.shape(U_K)[2]) if U_K is not None else 0
    rv = int(np.shape(U_V)[2]) if U_V is not None else 0
    U_K, U_V, C_K, C_V, K_raw, V_raw, k_new, v_new = (
        _arr(x, dt) for x in (U_K, U_V, C_K, C_V, K_raw, V_raw, k_new, v_new))
    nbl = _arr(num_beacons, np.dtype(np.int32))
    rwl = _arr(raw_len, np.dtype(np.int32))
    prob = _Problem(B, Hq, num_kv_heads, d, ncap, rk, rv, wcap, float(scale), float(rope_theta),
                    _DTYPE[dt])
    out = np.full((B, Hq, d), np.nan, dtype=np.float64)
    lse = np.full((B, Hq), np.nan, dtype=np.float64)
    k_app = np.full((B, num_kv_heads, d), np.nan, dtype=np.float64)
    if units is None:
        unit_arr, n_units = None, 0
    else:
        unit_arr = np.ascontiguousarray(np.asarray(units, dtype=np.int32).reshape(-1, 2))
        n_units = unit_arr.shape[0]

    def ptr(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    rc = load(library).slimkv_oracle_decode_ragged(
        ctypes.byref(prob), ptr(q), ptr(q_pos), ptr(U_K), ptr(U_V), ptr(C_K), ptr(C_V),
        ptr(K_raw), ptr(V_raw), ptr(nbl), ptr(rwl), ptr(k_new), ptr(v_new), ptr(unit_arr),
        n_units, ptr(out), ptr(lse), ptr(k_app), int(threads))
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    return out, lse, k_app


def decode_chunk(q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw, *, num_kv_heads: int, scale: float,
                 rope_theta: float, num_beacons=None, raw_len=None, k_new=None, v_new=None,
                 units=None, threads: int = 0, library: pathlib.Path = LIBRARY):
    """fp64 attention of a chunk of Q query tokens per sequence (speculative
    decoding, chunked prefill) over a ragged cache.

    q [B, Q, H_q, d]: token t of sequence b at position q_pos[b] + t.  The
    cache arrays, lengths and their clamping are those of ``decode_ragged``.
    ``k_new``, ``v_new`` ([B, Q, H_kv, d], both or neither): the chunk's
    tokens; token t's query attends over the live cache rows and new tokens
    0..t, each key rotated at its own position and rounded to the storage
    precision.  Returns (out [B, Q, H_q, d], lse [B, Q, H_q], k_app
    [B, Q, H_kv, d]) in float64 (k_app NaN without new tokens).
    """
    q = np.ascontiguousarray(q)
    dt = q.dtype
    if dt not in _DTYPE:
        raise TypeError(f"unsupported storage dtype {dt}")
    B, Q, Hq, d = q.shape
    q_pos = _arr(q_pos, np.dtype(np.int32))
    ncap = 0 if C_K is None else int(np.shape(C_K)[2])
    wcap = 0 if K_raw is None else int(np.shape(K_raw)[2])
    rk = int(np.shape(U_K)[2]) if U_K is not None else 0
    rv = int(np.shape(U_V)[2]) if U_V is not None else 0
    U_K, U_V, C_K, C_V, K_raw, V_raw, k_new, v_new = (
        _arr(x, dt) for x in (U_K, U_V, C_K, C_V, K_raw, V_raw, k_new, v_new))
    nbl = _arr(num_beacons, np.dtype(np.int32))
    rwl = _arr(raw_len, np.dtype(np.int32))
    prob = _Problem(B, Hq, num_kv_heads, d, ncap, rk, rv, wcap, float(scale), float(rope_theta),
                    _DTYPE[dt])
    out = np.full((B, Q, Hq, d), np.nan, dtype=np.float64)
    lse = np.full((B, Q, Hq), np.nan, dtype=np.float64)
    k_app = np.full((B, Q, num_kv_heads, d), np.nan, dtype=np.float64)
    if units is None:
        unit_arr, n_units = None, 0
    else:
        unit_arr = np.ascontiguousarray(np.asarray(units, dtype=np.int32).reshape(-1, 2))
        n_units = unit_arr.shape[0]

    def ptr(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    rc = load(library).slimkv_oracle_decode_chunk(
        ctypes.byref(prob), int(Q), ptr(q), ptr(q_pos), ptr(U_K), ptr(U_V), ptr(C_K), ptr(C_V),
        ptr(K_raw), ptr(V_raw), ptr(nbl), ptr(rwl), ptr(k_new), ptr(v_new), ptr(unit_arr),
        n_units, ptr(out), ptr(lse), ptr(k_app), int(threads))
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    return out, lse, k_app


def decode_alibi(q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw, *, beacon_pos, slopes,
                 num_kv_heads: int, scale: float, units=None, threads: int = 0,
                 library: pathlib.Path = LIBRARY):
    """fp64 latent decode attention of an ALiBi backbone: no rotation; score
    j gets -slopes[h_q] * (q_pos - k_pos) after the scaled product, with
    beacon j at beacon_pos[j] ([N_b] int32) and raw row t at
    q_pos - W + 1 + t.  Arrays and the result as for ``decode``; slopes
    [H_q] float64."""
    q = np.ascontiguousarray(q)
    dt = q.dtype
    if dt not in _DTYPE:
        raise TypeError(f"unsupported storage dtype {dt}")
    B, Hq, d = q.shape
    q_pos = _arr(q_pos, np.dtype(np.int32))
    nb = 0 if C_K is None else int(np.shape(C_K)[2])
    w = 0 if K_raw is None else int(np.shape(K_raw)[2])
    rk = int(np.shape(U_K)[2]) if U_K is not None else 0
    rv = int(np.shape(U_V)[2]) if U_V is not None else 0
    U_K, U_V, C_K, C_V, K_raw, V_raw = (_arr(x, dt) for x in (U_K, U_V, C_K, C_V, K_raw, V_raw))
    bp = _arr(beacon_pos, np.dtype(np.int32)) if nb else None
    sl = np.ascontiguousarray(slopes, dtype=np.float64)
    if sl.shape != (Hq,):
        raise ValueError("slopes must have one entry per query head")
    prob = _Problem(B, Hq, num_kv_heads, d, nb, rk, rv, w, float(scale), 10000.0, _DTYPE[dt])
    out = np.full((B, Hq, d), np.nan, dtype=np.float64)
    lse = np.full((B, Hq), np.nan, dtype=np.float64)
    if units is None:
        unit_arr, n_units = None, 0
    else:
        unit_arr = np.ascontiguousarray(np.asarray(units, dtype=np.int32).reshape(-1, 2))
        n_units = unit_arr.shape[0]

    def ptr(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    rc = load(library).slimkv_oracle_decode_alibi(
        ctypes.byref(prob), ptr(q), ptr(q_pos), ptr(U_K), ptr(U_V), ptr(C_K), ptr(C_V),
        ptr(K_raw), ptr(V_raw), ptr(bp), ptr(sl), ptr(unit_arr), n_units, ptr(out), ptr(lse),
        int(threads))
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    return out, lse


def decode_chunk_alibi(q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw, *, beacon_pos, slopes,
                       num_kv_heads: int, scale: float, num_beacons=None, raw_len=None,
                       k_new=None, v_new=None, units=None, threads: int = 0,
                       library: pathlib.Path = LIBRARY):
    """fp64 ALiBi attention of a serving step: ``decode_chunk``'s ragged
    cache, new tokens and Q query tokens per sequence, scored as in
    ``decode_alibi`` (nothing rotated; score gets -slopes[h_q] * (q_pos_t -
    k_pos)).  Positions: query token t at q_pos[b] + t, beacon j at
    beacon_pos[j], new token u at q_pos[b] + u, live raw row i at
    q_pos[b] - w_b + i with new tokens and q_pos[b] - w_b + 1 + i without.
    q [B, Q, H_q, d] (a 3-d q is one token per sequence).  Returns (out, lse,
    k_app) shaped [B, Q, H_q, d], [B, Q, H_q], [B, Q, H_kv, d] (squeezed to
    3-d / 2-d when q was 3-d)."""
    q = np.ascontiguousarray(q)
    squeeze = q.ndim == 3
    if squeeze:
        q = q[:, None]
        k_new = None if k_new is None else np.ascontiguousarray(k_new)[:, None]
        v_new = None if v_new is None else np.ascontiguousarray(v_new)[:, None]
    dt = q.dtype
    if dt not in _DTYPE:
        raise TypeError(f"unsupported storage dtype {dt}")
    B, Q, Hq, d = q.shape
    q_pos = _arr(q_pos, np.dtype(np.int32))
    ncap = 0 if C_K is None else int(np.shape(C_K)[2])
    wcap = 0 if K_raw is None else int(np.shape(K_raw)[2])
    rk = int(np.shape(U_K)[2]) if U_K is not None else 0
    rv = int(np.shape(U_V)[2]) if U_V is not None else 0
    U_K, U_V, C_K, C_V, K_raw, V_raw, k_new, v_new = (
        _arr(x, dt) for x in (U_K, U_V, C_K, C_V, K_raw, V_raw, k_new, v_new))
    nbl = _arr(num_beacons, np.dtype(np.int32))
    rwl = _arr(raw_len, np.dtype(np.int32))
    bp = _arr(beacon_pos, np.dtype(np.int32)) if ncap else None
    sl = np.ascontiguousarray(slopes, dtype=np.float64)
    if sl.shape != (Hq,):
        raise ValueError("slopes must have one entry per query head")
    prob = _Problem(B, Hq, num_kv_heads, d, ncap, rk, rv, wcap, float(scale), 10000.0, _DTYPE[dt])
    out = np.full((B, Q, Hq, d), np.nan, dtype=np.float64)
    lse = np.full((B, Q, Hq), np.nan, dtype=np.float64)
    k_app = np.full((B, Q, num_kv_heads, d), np.nan, dtype=np.float64)
    if units is None:
        unit_arr, n_units = None, 0
    else:
        unit_arr = np.ascontiguousarray(np.asarray(units, dtype=np.int32).reshape(-1, 2))
        n_units = unit_arr.shape[0]

    def ptr(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    rc = load(library).slimkv_oracle_decode_chunk_alibi(
        ctypes.byref(prob), int(Q), ptr(q), ptr(q_pos), ptr(U_K), ptr(U_V), ptr(C_K), ptr(C_V),
        ptr(K_raw), ptr(V_raw), ptr(nbl), ptr(rwl), ptr(k_new), ptr(v_new), ptr(bp), ptr(sl),
        ptr(unit_arr), n_units, ptr(out), ptr(lse), ptr(k_app), int(threads))
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    if squeeze:
        return out[:, 0], lse[:, 0], k_app[:, 0]
    return out, lse, k_app


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
