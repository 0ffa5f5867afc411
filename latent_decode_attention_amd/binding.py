"""ctypes binding of libslimkv.so, with the C ABI's names.

Argument marshalling only: tensors are torch tensors in device memory, whose
pointers and the current HIP stream are handed to the library; every step of
the attention runs in the library's HIP kernels.  There is no fallback: if
the library is missing, loading fails with an error that says how to build
it.
"""

from __future__ import annotations

import ctypes
import pathlib

import torch

LIBRARY = pathlib.Path(__file__).resolve().parent / "libslimkv.so"

SLIMKV_FP32, SLIMKV_BF16 = 0, 1
SLIMKV_OP_LATENT, SLIMKV_OP_RECONSTRUCT, SLIMKV_OP_FULL_KV, SLIMKV_OP_LATENT_RAGGED = 0, 1, 2, 3
SLIMKV_FLAG_DYNAMIC_TILES = 1
SLIMKV_FLAG_CHECK_WORKSPACE = 2
STATUS_NAMES = {0: "SLIMKV_OK", 1: "SLIMKV_ERR_NULL", 2: "SLIMKV_ERR_SHAPE",
                3: "SLIMKV_ERR_UNSUPPORTED", 4: "SLIMKV_ERR_WORKSPACE", 5: "SLIMKV_ERR_ALIGN",
                6: "SLIMKV_ERR_ALIAS", 7: "SLIMKV_ERR_HIP"}

EXPORTS = ("slimkv_workspace_bytes", "slimkv_decode_attn", "slimkv_decode_attn_noalloc",
           "slimkv_decode_attn_ragged",
           "slimkv_decode_attn_paged", "slimkv_chunk_workspace_bytes", "slimkv_decode_attn_chunk",
           "slimkv_decode_attn_chunk_paged", "slimkv_decode_attn_alibi",
           "slimkv_decode_attn_ragged_alibi", "slimkv_decode_attn_paged_alibi",
           "slimkv_decode_attn_chunk_alibi", "slimkv_decode_attn_chunk_paged_alibi",
           "slimkv_reconstruct_attn", "slimkv_reconstruct_rope_attn", "full_kv_attn",
           "slimkv_set_kernel_events",
           "slimkv_workspace_status", "slimkv_status_string", "slimkv_last_error",
           "slimkv_abi_version",
           "slimkv_bench_stream_read", "slimkv_bench_flush")


class slimkv_problem(ctypes.Structure):  # noqa: N801  (C name)
    """Mirror of ``slimkv_problem`` in include/slimkv.h (56 bytes)."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("num_beacons", ctypes.c_int32),
        ("rank_k", ctypes.c_int32),
        ("rank_v", ctypes.c_int32),
        ("raw_window", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("num_splits", ctypes.c_int32),
        ("flags", ctypes.c_int32),
    ]


assert ctypes.sizeof(slimkv_problem) == 56


class slimkv_pages(ctypes.Structure):  # noqa: N801  (C name)
    """Mirror of ``slimkv_pages`` in include/slimkv.h (40 bytes); the tables
    are device pointers."""

    _fields_ = [
        ("page_rows", ctypes.c_int32),
        ("beacon_pages", ctypes.c_int32),
        ("raw_pages", ctypes.c_int32),
        ("beacon_table_width", ctypes.c_int32),
        ("raw_table_width", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("beacon_table", ctypes.c_void_p),
        ("raw_table", ctypes.c_void_p),
    ]


assert ctypes.sizeof(slimkv_pages) == 40


class slimkv_alibi(ctypes.Structure):  # noqa: N801  (C name)
    """Mirror of ``slimkv_alibi`` in include/slimkv.h (16 bytes); slopes is a
    device pointer."""

    _fields_ = [
        ("slopes", ctypes.c_void_p),
        ("beacon_first", ctypes.c_int32),
        ("beacon_stride", ctypes.c_int32),
    ]


assert ctypes.sizeof(slimkv_alibi) == 16


class SlimKVError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")


_lib = None


def load_library(path: pathlib.Path | None = None) -> ctypes.CDLL:
    """Load libslimkv.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = pathlib.Path(path) if path else LIBRARY
    if not p.exists():
        raise RuntimeError(f"{p} is missing: build it with "
                           "`python -m latent_decode_attention_amd.build`")
    lib = ctypes.CDLL(str(p))
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    prob = ctypes.POINTER(slimkv_problem)
    lib.slimkv_workspace_bytes.argtypes = [prob, ctypes.c_int]
    lib.slimkv_workspace_bytes.restype = sz
    lib.slimkv_decode_attn.argtypes = [prob] + [vp] * 10 + [vp, sz, vp]
    lib.slimkv_decode_attn.restype = ctypes.c_int
    lib.slimkv_decode_attn_noalloc.argtypes = [prob] + [vp] * 10 + [vp]
    lib.slimkv_decode_attn_noalloc.restype = ctypes.c_int
    lib.slimkv_decode_attn_ragged.argtypes = [prob] + [vp] * 14 + [vp, sz, vp]
    lib.slimkv_decode_attn_ragged.restype = ctypes.c_int
    lib.slimkv_decode_attn_paged.argtypes = [prob, ctypes.POINTER(slimkv_pages)] + [vp] * 14 + [
        vp, sz, vp]
    lib.slimkv_decode_attn_paged.restype = ctypes.c_int
    lib.slimkv_decode_attn_alibi.argtypes = [prob] + [vp] * 9 + [ctypes.c_int32, ctypes.c_int32] + [
        vp, vp, vp, sz, vp]
    lib.slimkv_decode_attn_alibi.restype = ctypes.c_int
    al = ctypes.POINTER(slimkv_alibi)
    pgs = ctypes.POINTER(slimkv_pages)
    lib.slimkv_decode_attn_ragged_alibi.argtypes = [prob, al] + [vp] * 14 + [vp, sz, vp]
    lib.slimkv_decode_attn_ragged_alibi.restype = ctypes.c_int
    lib.slimkv_decode_attn_paged_alibi.argtypes = [prob, pgs, al] + [vp] * 14 + [vp, sz, vp]
    lib.slimkv_decode_attn_paged_alibi.restype = ctypes.c_int
    lib.slimkv_decode_attn_chunk_alibi.argtypes = [prob, al, ctypes.c_int32] + [vp] * 14 + [vp, sz, vp]
    lib.slimkv_decode_attn_chunk_alibi.restype = ctypes.c_int
    lib.slimkv_decode_attn_chunk_paged_alibi.argtypes = [prob, pgs, al, ctypes.c_int32] + [vp] * 14 + [
        vp, sz, vp]
    lib.slimkv_decode_attn_chunk_paged_alibi.restype = ctypes.c_int
    lib.slimkv_chunk_workspace_bytes.argtypes = [prob, ctypes.c_int32]
    lib.slimkv_chunk_workspace_bytes.restype = sz
    lib.slimkv_decode_attn_chunk.argtypes = [prob, ctypes.c_int32] + [vp] * 14 + [vp, sz, vp]
    lib.slimkv_decode_attn_chunk.restype = ctypes.c_int
    lib.slimkv_decode_attn_chunk_paged.argtypes = [prob, ctypes.POINTER(slimkv_pages),
                                                   ctypes.c_int32] + [vp] * 14 + [vp, sz, vp]
    lib.slimkv_decode_attn_chunk_paged.restype = ctypes.c_int
    lib.slimkv_reconstruct_attn.argtypes = [prob] + [vp] * 10 + [vp, sz, vp]
    lib.slimkv_reconstruct_attn.restype = ctypes.c_int
    lib.slimkv_reconstruct_rope_attn.argtypes = [prob] + [vp] * 11 + [vp, sz, vp]
    lib.slimkv_reconstruct_rope_attn.restype = ctypes.c_int
    lib.full_kv_attn.argtypes = [prob] + [vp] * 6 + [vp, sz, vp]
    lib.full_kv_attn.restype = ctypes.c_int
    lib.slimkv_status_string.argtypes = [ctypes.c_int]
    lib.slimkv_status_string.restype = ctypes.c_char_p
    lib.slimkv_last_error.argtypes = []
    lib.slimkv_last_error.restype = ctypes.c_char_p
    lib.slimkv_set_kernel_events.argtypes = [vp, vp]
    lib.slimkv_set_kernel_events.restype = ctypes.c_int
    lib.slimkv_workspace_status.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32)]
    lib.slimkv_workspace_status.restype = ctypes.c_int
    lib.slimkv_abi_version.argtypes = []
    lib.slimkv_abi_version.restype = ctypes.c_int32
    lib.slimkv_bench_stream_read.argtypes = [vp, sz, ctypes.c_int32, ctypes.c_int32, vp, vp]
    lib.slimkv_bench_stream_read.restype = ctypes.c_int
    lib.slimkv_bench_flush.argtypes = [vp, sz, ctypes.c_uint32, vp]
    lib.slimkv_bench_flush.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def make_problem(*, batch, num_q_heads, num_kv_heads, num_beacons, rank_k, rank_v, raw_window,
                 scale, rope_theta, dtype, head_dim=128, num_splits=0, flags=0) -> slimkv_problem:
    dt = {"fp32": SLIMKV_FP32, "bf16": SLIMKV_BF16, torch.float32: SLIMKV_FP32,
          torch.bfloat16: SLIMKV_BF16}.get(dtype, dtype)
    return slimkv_problem(batch, num_q_heads, num_kv_heads, head_dim, num_beacons, rank_k, rank_v,
                          raw_window, scale, dt, rope_theta, num_splits, flags)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a torch.Tensor or None, got {type(t).__name__}")
    if not t.is_contiguous():
        raise TypeError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(lib, status: int) -> None:
    if status != 0:
        raise SlimKVError(status, lib.slimkv_last_error().decode())


def slimkv_workspace_bytes(problem: slimkv_problem, op: int) -> int:
    lib = load_library()
    n = lib.slimkv_workspace_bytes(ctypes.byref(problem), op)
    if n == 0:
        raise SlimKVError(2, lib.slimkv_last_error().decode())
    return int(n)


def slimkv_decode_attn(problem, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw, out, lse, workspace,
                       stream=None) -> None:
    lib = load_library()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib, lib.slimkv_decode_attn(
        ctypes.byref(problem), _ptr(q), _ptr(q_pos), _ptr(U_K), _ptr(U_V), _ptr(C_K), _ptr(C_V),
        _ptr(K_raw), _ptr(V_raw), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
        _stream(stream)))


def slimkv_decode_attn_noalloc(problem, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw, out, lse,
                               stream=None) -> None:
    lib = load_library()
    _check(lib, lib.slimkv_decode_attn_noalloc(
        ctypes.byref(problem), _ptr(q), _ptr(q_pos), _ptr(U_K), _ptr(U_V), _ptr(C_K), _ptr(C_V),
        _ptr(K_raw), _ptr(V_raw), _ptr(out), _ptr(lse), _stream(stream)))


def slimkv_decode_attn_ragged(problem, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw, num_beacons,
                              raw_len, k_new, v_new, out, lse, workspace, stream=None) -> None:
    lib = load_library()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib, lib.slimkv_decode_attn_ragged(
        ctypes.byref(problem), _ptr(q), _ptr(q_pos), _ptr(U_K), _ptr(U_V), _ptr(C_K), _ptr(C_V),
        _ptr(K_raw), _ptr(V_raw), _ptr(num_beacons), _ptr(raw_len), _ptr(k_new), _ptr(v_new),
        _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def make_pages(*, page_rows, beacon_table=None, raw_table=None, beacon_pages=0,
               raw_pages=0) -> slimkv_pages:
    """slimkv_pages from int32 tables [B, width] (device tensors or None)."""
    def width(t):
        if t is None:
            return 0
        if t.dtype != torch.int32 or t.dim() != 2:
            raise TypeError("page tables are int32 [B, width] tensors")
        return t.shape[1]
    return slimkv_pages(page_rows, beacon_pages, raw_pages, width(beacon_table), width(raw_table),
                        0, _ptr(beacon_table), _ptr(raw_table))


def slimkv_decode_attn_paged(problem, pages, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw,
                             num_beacons, raw_len, k_new, v_new, out, lse, workspace,
                             stream=None) -> None:
    lib = load_library()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib, lib.slimkv_decode_attn_paged(
        ctypes.byref(problem), ctypes.byref(pages) if pages is not None else None, _ptr(q),
        _ptr(q_pos), _ptr(U_K), _ptr(U_V), _ptr(C_K), _ptr(C_V), _ptr(K_raw), _ptr(V_raw),
        _ptr(num_beacons), _ptr(raw_len), _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(lse),
        _ptr(workspace), ws_bytes, _stream(stream)))


def slimkv_decode_attn_alibi(problem, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw, slopes,
                             beacon_first, beacon_stride, out, lse, workspace, stream=None) -> None:
    lib = load_library()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib, lib.slimkv_decode_attn_alibi(
        ctypes.byref(problem), _ptr(q), _ptr(q_pos), _ptr(U_K), _ptr(U_V), _ptr(C_K), _ptr(C_V),
        _ptr(K_raw), _ptr(V_raw), _ptr(slopes), int(beacon_first), int(beacon_stride), _ptr(out),
        _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def make_alibi(slopes, beacon_first: int, beacon_stride: int) -> slimkv_alibi:
    """slimkv_alibi from a float32 [H_q] device tensor of slopes."""
    if slopes.dtype != torch.float32:
        raise TypeError("slopes must be float32")
    return slimkv_alibi(_ptr(slopes), int(beacon_first), int(beacon_stride))


def slimkv_decode_attn_ragged_alibi(problem, alibi, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw,
                                    num_beacons, raw_len, k_new, v_new, out, lse, workspace,
                                    stream=None) -> None:
    lib = load_library()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib, lib.slimkv_decode_attn_ragged_alibi(
        ctypes.byref(problem), ctypes.byref(alibi) if alibi is not None else None, _ptr(q),
        _ptr(q_pos), _ptr(U_K), _ptr(U_V), _ptr(C_K), _ptr(C_V), _ptr(K_raw), _ptr(V_raw),
        _ptr(num_beacons), _ptr(raw_len), _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(lse),
        _ptr(workspace), ws_bytes, _stream(stream)))


def slimkv_decode_attn_paged_alibi(problem, pages, alibi, q, q_pos, U_K, U_V, C_K, C_V, K_raw,
                                   V_raw, num_beacons, raw_len, k_new, v_new, out, lse, workspace,
                                   stream=None) -> None:
    lib = load_library()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib, lib.slimkv_decode_attn_paged_alibi(
        ctypes.byref(problem), ctypes.byref(pages) if pages is not None else None,
        ctypes.byref(alibi) if alibi is not None else None, _ptr(q), _ptr(q_pos), _ptr(U_K),
        _ptr(U_V), _ptr(C_K), _ptr(C_V), _ptr(K_raw), _ptr(V_raw), _ptr(num_beacons),
        _ptr(raw_len), _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
        _stream(stream)))


def slimkv_decode_attn_chunk_alibi(problem, alibi, num_tokens, q, q_pos, U_K, U_V, C_K, C_V,
                                   K_raw, V_raw, num_beacons, raw_len, k_new, v_new, out, lse,
                                   workspace, stream=None) -> None:
    lib = load_library()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib, lib.slimkv_decode_attn_chunk_alibi(
        ctypes.byref(problem), ctypes.byref(alibi) if alibi is not None else None,
        int(num_tokens), _ptr(q), _ptr(q_pos), _ptr(U_K), _ptr(U_V), _ptr(C_K), _ptr(C_V),
        _ptr(K_raw), _ptr(V_raw), _ptr(num_beacons), _ptr(raw_len), _ptr(k_new), _ptr(v_new),
        _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def slimkv_decode_attn_chunk_paged_alibi(problem, pages, alibi, num_tokens, q, q_pos, U_K, U_V,
                                         C_K, C_V, K_raw, V_raw, num_beacons, raw_len, k_new,
                                         v_new, out, lse, workspace, stream=None) -> None:
    lib = load_library()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib, lib.slimkv_decode_attn_chunk_paged_alibi(
        ctypes.byref(problem), ctypes.byref(pages) if pages is not None else None,
        ctypes.byref(alibi) if alibi is not None else None, int(num_tokens), _ptr(q),
        _ptr(q_pos), _ptr(U_K), _ptr(U_V), _ptr(C_K), _ptr(C_V), _ptr(K_raw), _ptr(V_raw),
        _ptr(num_beacons), _ptr(raw_len), _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(lse),
        _ptr(workspace), ws_bytes, _stream(stream)))


def slimkv_chunk_workspace_bytes(problem: slimkv_problem, num_tokens: int) -> int:
    lib = load_library()
    n = lib.slimkv_chunk_workspace_bytes(ctypes.byref(problem), int(num_tokens))
    if n == 0:
        raise SlimKVError(2, lib.slimkv_last_error().decode())
    return int(n)


def slimkv_decode_attn_chunk(problem, num_tokens, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw,
                             num_beacons, raw_len, k_new, v_new, out, lse, workspace,
                             stream=None) -> None:
    lib = load_library()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib, lib.slimkv_decode_attn_chunk(
        ctypes.byref(problem), int(num_tokens), _ptr(q), _ptr(q_pos), _ptr(U_K), _ptr(U_V),
        _ptr(C_K), _ptr(C_V), _ptr(K_raw), _ptr(V_raw), _ptr(num_beacons), _ptr(raw_len),
        _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
        _stream(stream)))


def slimkv_decode_attn_chunk_paged(problem, pages, num_tokens, q, q_pos, U_K, U_V, C_K, C_V,
                                   K_raw, V_raw, num_beacons, raw_len, k_new, v_new, out, lse,
                                   workspace, stream=None) -> None:
    lib = load_library()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib, lib.slimkv_decode_attn_chunk_paged(
        ctypes.byref(problem), ctypes.byref(pages) if pages is not None else None,
        int(num_tokens), _ptr(q), _ptr(q_pos), _ptr(U_K), _ptr(U_V), _ptr(C_K), _ptr(C_V),
        _ptr(K_raw), _ptr(V_raw), _ptr(num_beacons), _ptr(raw_len), _ptr(k_new), _ptr(v_new),
        _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def slimkv_reconstruct_attn(problem, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw, out, lse,
                            workspace, stream=None) -> None:
    lib = load_library()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib, lib.slimkv_reconstruct_attn(
        ctypes.byref(problem), _ptr(q), _ptr(q_pos), _ptr(U_K), _ptr(U_V), _ptr(C_K), _ptr(C_V),
        _ptr(K_raw), _ptr(V_raw), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
        _stream(stream)))


def slimkv_reconstruct_rope_attn(problem, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw,
                                 beacon_pos, out, lse, workspace, stream=None) -> None:
    lib = load_library()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib, lib.slimkv_reconstruct_rope_attn(
        ctypes.byref(problem), _ptr(q), _ptr(q_pos), _ptr(U_K), _ptr(U_V), _ptr(C_K), _ptr(C_V),
        _ptr(K_raw), _ptr(V_raw), _ptr(beacon_pos), _ptr(out), _ptr(lse), _ptr(workspace),
        ws_bytes, _stream(stream)))


def full_kv_attn(problem, q, q_pos, K, V, out, lse, workspace, stream=None) -> None:
    lib = load_library()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib, lib.full_kv_attn(
        ctypes.byref(problem), _ptr(q), _ptr(q_pos), _ptr(K), _ptr(V), _ptr(out), _ptr(lse),
        _ptr(workspace), ws_bytes, _stream(stream)))


def slimkv_set_kernel_events(start, stop) -> None:
    """Time the next call's attention kernel with two torch.cuda.Event (or raw
    hipEvent_t handles); None, None clears a pending pair."""
    lib = load_library()
    def handle(e):
        if e is None:
            return None
        if isinstance(e, torch.cuda.Event):
            if not e.cuda_event:  # torch creates the HIP event on first record
                e.record()
            return e.cuda_event
        return int(e)
    _check(lib, lib.slimkv_set_kernel_events(handle(start), handle(stop)))


def slimkv_status_string(status: int) -> str:
    return load_library().slimkv_status_string(status).decode()


def slimkv_last_error() -> str:
    return load_library().slimkv_last_error().decode()


def slimkv_workspace_status(workspace) -> int:
    """The workspace's status word (bit 0: a call made with
    SLIMKV_FLAG_CHECK_WORKSPACE found its counters or flags not at zero).
    Synchronous: waits for the device."""
    lib = load_library()
    word = ctypes.c_uint32(0)
    _check(lib, lib.slimkv_workspace_status(_ptr(workspace), ctypes.byref(word)))
    return int(word.value)


def slimkv_abi_version() -> int:
    return int(load_library().slimkv_abi_version())


def _check_bench(status: int, what: str) -> None:
    if status != 0:
        raise SlimKVError(status, what)


def slimkv_bench_stream_read(src, sink, *, in_flight: int = 4, workgroups: int = 0,
                             nbytes: int | None = None, stream=None) -> None:
    """Stream ``nbytes`` (default: all) of the tensor ``src`` once through the
    plain read kernel; its checksum goes to ``sink`` (a 1-element int32 or
    uint32 tensor)."""
    lib = load_library()
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    _check_bench(lib.slimkv_bench_stream_read(_ptr(src), n, int(in_flight), int(workgroups),
                                              _ptr(sink), _stream(stream)),
                 f"slimkv_bench_stream_read({n} bytes, in_flight {in_flight})")


def slimkv_bench_flush(buf, seed: int = 0, stream=None) -> None:
    """Overwrite the whole of ``buf`` (a contiguous device tensor)."""
    lib = load_library()
    n = buf.numel() * buf.element_size()
    _check_bench(lib.slimkv_bench_flush(_ptr(buf), n, int(seed) & 0xffffffff, _stream(stream)),
                 f"slimkv_bench_flush({n} bytes)")
