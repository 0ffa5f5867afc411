"""The C ABI without a GPU: exported symbols, struct layout, and every
argument check (they all run before any HIP call, so they are safe here)."""

import ctypes
import pathlib
import re

import pytest

import latent_decode_attention_amd as lda
from latent_decode_attention_amd import binding

INCLUDE = pathlib.Path(__file__).resolve().parents[1] / "include"
HEADER = INCLUDE / "slimkv.h"
OK, NULL, SHAPE, UNSUP, WS, ALIGN, ALIAS = 0, 1, 2, 3, 4, 5, 6


def header_functions():
    """Every function declared in include/*.h."""
    names = set()
    for h in sorted(INCLUDE.glob("*.h")):
        text = re.sub(r"/\*.*?\*/", "", h.read_text(), flags=re.S)
        names |= set(re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    return lda.load_library()


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert set(names) == set(binding.EXPORTS), names
    for name in names:
        assert hasattr(lib, name), f"{name} not exported"


def test_problem_struct_layout():
    text = HEADER.read_text()
    body = re.search(r"typedef struct slimkv_problem \{(.*?)\} slimkv_problem;", text, re.S).group(1)
    fields = re.findall(r"^\s*(int32_t|float|double)\s+(\w+);", body, re.M)
    assert [f for _, f in fields] == [f for f, _ in binding.slimkv_problem._fields_]
    assert ctypes.sizeof(binding.slimkv_problem) == 56
    assert binding.slimkv_problem.rope_theta.offset == 40


def test_version_and_status_strings(lib):
    assert lda.slimkv_abi_version() == 9
    for code in range(8):
        assert lda.slimkv_status_string(code)
    assert lda.slimkv_status_string(99) == "unknown status"


def _problem(**over):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, num_beacons=64, rank_k=32, rank_v=32,
                raw_window=32, scale=0.088, rope_theta=5e5, dtype="bf16")
    base.update(over)
    return lda.make_problem(**base)


def _call(lib, prob, *, op=0, ptrs=None, ws_bytes=1 << 30):
    """Call an entry point with fake device addresses (never dereferenced:
    every case here fails validation before any HIP call)."""
    p = dict(q=0x100000, q_pos=0x200000, U_K=0x300000, U_V=0x400000, C_K=0x1000000,
             C_V=0x2000000, K_raw=0x3000000, V_raw=0x4000000, out=0x5000000, lse=0x6000000,
             ws=0x7000000)
    p.update(ptrs or {})
    v = {k: (None if x is None else ctypes.c_void_p(x)) for k, x in p.items()}
    pp = ctypes.byref(prob) if prob is not None else None
    if op == 2:
        return lib.full_kv_attn(pp, v["q"], v["q_pos"], v["K_raw"], v["V_raw"], v["out"],
                                v["lse"], v["ws"], ws_bytes, None)
    fn = lib.slimkv_decode_attn if op == 0 else lib.slimkv_reconstruct_attn
    return fn(pp, v["q"], v["q_pos"], v["U_K"], v["U_V"], v["C_K"], v["C_V"], v["K_raw"],
              v["V_raw"], v["out"], v["lse"], v["ws"], ws_bytes, None)


@pytest.mark.parametrize("over,status", [
    (dict(num_q_heads=7), SHAPE),
    (dict(num_q_heads=32, num_kv_heads=2), UNSUP),  # group 16 > 8
    (dict(head_dim=64), UNSUP),
    (dict(num_beacons=0, raw_window=0), SHAPE),
    (dict(num_beacons=-1), SHAPE),
    (dict(rank_k=40), UNSUP),
    (dict(rank_v=144), UNSUP),
    (dict(rank_k=0), UNSUP),
    (dict(dtype=5), UNSUP),
    (dict(scale=0.0), SHAPE),
    (dict(scale=float("inf")), SHAPE),
    (dict(rope_theta=1.0), SHAPE),
    (dict(rope_theta=float("nan")), SHAPE),
    (dict(batch=0), SHAPE),
    (dict(num_splits=-3), SHAPE),
    (dict(num_beacons=1 << 25), UNSUP),
])
def test_shape_errors(lib, over, status):
    prob = _problem(**over)
    assert _call(lib, prob) == status
    assert lda.slimkv_last_error()
    assert lib.slimkv_workspace_bytes(ctypes.byref(prob), 0) == 0


def test_unknown_flag_bits_rejected(lib):
    prob = _problem()
    prob.flags = 4
    assert _call(lib, prob) == SHAPE
    assert "flag" in lda.slimkv_last_error()
    assert lib.slimkv_workspace_bytes(ctypes.byref(prob), 0) == 0
    for f in (lda.SLIMKV_FLAG_DYNAMIC_TILES, lda.SLIMKV_FLAG_CHECK_WORKSPACE,
              lda.SLIMKV_FLAG_DYNAMIC_TILES | lda.SLIMKV_FLAG_CHECK_WORKSPACE):
        prob.flags = f
        assert lib.slimkv_workspace_bytes(ctypes.byref(prob), 0) > 0


def test_workspace_status_checks(lib):
    """slimkv_workspace_status rejects NULL and misaligned workspaces
    before it touches the device."""
    word = ctypes.c_uint32(7)
    assert lib.slimkv_workspace_status(None, ctypes.byref(word)) == NULL
    assert lib.slimkv_workspace_status(ctypes.c_void_p(0x100000), None) == NULL
    assert lib.slimkv_workspace_status(ctypes.c_void_p(0x100004), ctypes.byref(word)) == ALIGN
    assert word.value == 7


def test_null_problem(lib):
    assert _call(lib, None) == NULL


@pytest.mark.parametrize("name", ["q", "q_pos", "U_K", "U_V", "C_K", "C_V", "K_raw", "V_raw",
                                  "out", "ws"])
def test_null_pointers(lib, name):
    assert _call(lib, _problem(), ptrs={name: None}) == NULL
    assert name.replace("ws", "workspace") in lda.slimkv_last_error()


def test_optional_pointers_follow_sizes(lib):
    # no beacons: U/C may be NULL; no raw rows: K_raw/V_raw may be NULL.  The
    # call then fails later, on the workspace size, not on a NULL pointer.
    prob = _problem(num_beacons=0)
    st = _call(lib, prob, ptrs=dict(U_K=None, U_V=None, C_K=None, C_V=None), ws_bytes=16)
    assert st == WS
    prob = _problem(raw_window=0)
    assert _call(lib, prob, ptrs=dict(K_raw=None, V_raw=None), ws_bytes=16) == WS


def test_workspace_too_small(lib):
    prob = _problem()
    need = lib.slimkv_workspace_bytes(ctypes.byref(prob), 0)
    assert need > 0
    assert _call(lib, prob, ws_bytes=need - 1) == WS
    assert str(need) in lda.slimkv_last_error()


@pytest.mark.parametrize("name", ["q", "U_K", "C_K", "V_raw", "ws"])
def test_misaligned(lib, name):
    base = {"q": 0x100000, "U_K": 0x300000, "C_K": 0x1000000, "V_raw": 0x4000000, "ws": 0x7000000}
    assert _call(lib, _problem(), ptrs={name: base[name] + 8}) == ALIGN


def test_misaligned_q_pos(lib):
    assert _call(lib, _problem(), ptrs={"q_pos": 0x200002}) == ALIGN


@pytest.mark.parametrize("ptrs", [
    dict(out=0x1000000 + 64),   # out inside C_K
    dict(lse=0x5000000 + 16),   # lse inside out
    dict(ws=0x3000000),         # workspace on K_raw
    dict(out=0x200000),         # out on q_pos
])
def test_aliasing(lib, ptrs):
    assert _call(lib, _problem(), ptrs=ptrs) == ALIAS


def test_full_kv_needs_no_beacons(lib):
    assert _call(lib, _problem(num_beacons=64), op=2) == SHAPE
    assert _call(lib, _problem(num_beacons=0), op=2, ws_bytes=16) == WS


def test_workspace_bytes_by_op(lib):
    prob = _problem()
    lat = lib.slimkv_workspace_bytes(ctypes.byref(prob), 0)
    rec = lib.slimkv_workspace_bytes(ctypes.byref(prob), 1)
    # the reconstruction path also holds the rebuilt beacon keys and values
    assert rec - lat >= 2 * 2 * 2 * 64 * 128 * 2 - 32 * 8 * 2 * 4
    assert lib.slimkv_workspace_bytes(ctypes.byref(prob), 7) == 0
    assert lib.slimkv_workspace_bytes(None, 0) == 0


def test_workspace_does_not_depend_on_split_choice(lib):
    # sized for the largest chunk count, so one workspace serves any split
    sizes = {lib.slimkv_workspace_bytes(ctypes.byref(_problem(num_splits=s)), 0)
             for s in (0, 1, 4, 64, 1000)}
    assert len(sizes) == 1


def _call_ragged(lib, prob, *, ptrs=None, ws_bytes=1 << 30):
    """slimkv_decode_attn_ragged with fake device addresses (every case
    fails validation before any HIP call)."""
    p = dict(q=0x100000, q_pos=0x200000, U_K=0x300000, U_V=0x400000, C_K=0x1000000,
             C_V=0x2000000, K_raw=0x3000000, V_raw=0x4000000, nb=0x210000, raw=0x220000,
             k_new=0x230000, v_new=0x240000, out=0x5000000, lse=0x6000000, ws=0x7000000)
    p.update(ptrs or {})
    v = {k: (None if x is None else ctypes.c_void_p(x)) for k, x in p.items()}
    pp = ctypes.byref(prob) if prob is not None else None
    return lib.slimkv_decode_attn_ragged(pp, v["q"], v["q_pos"], v["U_K"], v["U_V"], v["C_K"],
                                         v["C_V"], v["K_raw"], v["V_raw"], v["nb"], v["raw"],
                                         v["k_new"], v["v_new"], v["out"], v["lse"], v["ws"],
                                         ws_bytes, None)


def test_ragged_checks(lib):
    ragged = lda.SLIMKV_OP_LATENT_RAGGED
    prob = _problem()
    need = lib.slimkv_workspace_bytes(ctypes.byref(prob), ragged)
    assert need > lib.slimkv_workspace_bytes(ctypes.byref(prob), 0)
    assert _call_ragged(lib, prob, ws_bytes=need - 1) == WS
    # only the new token: no cache rows at all is a valid ragged problem
    empty = _problem(num_beacons=0, raw_window=0)
    assert lib.slimkv_workspace_bytes(ctypes.byref(empty), ragged) > 0
    assert lib.slimkv_workspace_bytes(ctypes.byref(empty), 0) == 0
    assert _call_ragged(lib, empty, ptrs=dict(U_K=None, U_V=None, C_K=None, C_V=None,
                                               K_raw=None, V_raw=None), ws_bytes=16) == WS
    # the schedule is fixed; the lengths live in LDS
    prob.flags = lda.SLIMKV_FLAG_DYNAMIC_TILES
    assert _call_ragged(lib, prob) == UNSUP
    prob.flags = lda.SLIMKV_FLAG_CHECK_WORKSPACE
    assert lib.slimkv_workspace_bytes(ctypes.byref(prob), ragged) > 0
    prob.flags = 0
    assert _call_ragged(lib, _problem(batch=1025)) == UNSUP
    assert _call_ragged(lib, _problem(batch=1024), ws_bytes=16) == WS
    # the new token's key and value come together
    assert _call_ragged(lib, _problem(), ptrs=dict(v_new=None)) == NULL
    assert _call_ragged(lib, _problem(), ptrs=dict(k_new=None)) == NULL
    # lengths are optional; no new token is fine
    assert _call_ragged(lib, _problem(), ptrs=dict(nb=None, raw=None, k_new=None, v_new=None),
                        ws_bytes=16) == WS
    assert _call_ragged(lib, _problem(), ptrs=dict(raw=0x220002)) == ALIGN
    assert _call_ragged(lib, _problem(), ptrs=dict(k_new=0x230008)) == ALIGN
    # with a new token the raw window is written: it must not overlap inputs
    assert _call_ragged(lib, _problem(), ptrs=dict(k_new=0x3000000 + 256)) == ALIAS
    assert _call_ragged(lib, _problem(), ptrs=dict(ws=0x4000000)) == ALIAS
    # without one it is only read, and may not overlap the outputs either
    assert _call_ragged(lib, _problem(), ptrs=dict(k_new=None, v_new=None, out=0x3000000)) == ALIAS


def test_pages_struct_layout():
    text = HEADER.read_text()
    body = re.search(r"typedef struct slimkv_pages \{(.*?)\} slimkv_pages;", text, re.S).group(1)
    fields = re.findall(r"^\s*(?:const )?(int32_t\*?|int32_t)\s+(\w+);", body, re.M)
    assert [f for _, f in fields] == [f for f, _ in binding.slimkv_pages._fields_]
    assert ctypes.sizeof(binding.slimkv_pages) == 40
    assert binding.slimkv_pages.beacon_table.offset == 24


def _call_paged(lib, prob, pages, *, ptrs=None, ws_bytes=16):
    """slimkv_decode_attn_paged with fake device addresses (every case fails
    validation before any HIP call: at the latest, the 16-byte workspace is
    too small)."""
    p = dict(q=0x100000, q_pos=0x200000, U_K=0x300000, U_V=0x400000, C_K=0x1000000,
             C_V=0x2000000, K_raw=0x3000000, V_raw=0x4000000, nb=0x210000, raw=0x220000,
             k_new=0x230000, v_new=0x240000, out=0x5000000, lse=0x6000000, ws=0x7000000)
    p.update(ptrs or {})
    v = {k: (None if x is None else ctypes.c_void_p(x)) for k, x in p.items()}
    pg = ctypes.byref(pages) if pages is not None else None
    return lib.slimkv_decode_attn_paged(ctypes.byref(prob), pg, v["q"], v["q_pos"], v["U_K"],
                                        v["U_V"], v["C_K"], v["C_V"], v["K_raw"], v["V_raw"],
                                        v["nb"], v["raw"], v["k_new"], v["v_new"], v["out"],
                                        v["lse"], v["ws"], ws_bytes, None)


def _pages(**over):
    base = dict(page_rows=64, beacon_pages=4, raw_pages=4, beacon_table_width=1,
                raw_table_width=1, reserved=0, beacon_table=0x250000, raw_table=0x260000)
    base.update(over)
    return binding.slimkv_pages(**base)


def test_paged_checks(lib):
    prob = _problem()  # 64 beacons, 32 raw rows: one page each at 64 rows a page
    assert _call_paged(lib, prob, _pages()) == WS  # every check passes; workspace too small
    assert _call_paged(lib, prob, None) == NULL
    for rows in (32, 96, 1 << 17, 0, -64):
        assert _call_paged(lib, prob, _pages(page_rows=rows)) == SHAPE, rows
    # the largest page (beacon pools of one page, 8 MiB each here)
    assert _call_paged(lib, _problem(raw_window=0),
                       _pages(page_rows=1 << 16, beacon_pages=1, raw_table=None, raw_pages=0),
                       ptrs=dict(K_raw=None, V_raw=None)) == WS
    # pools are pages x H_kv x page_rows x width: 32 pages of 2 x 4096 x 32 x 2 B end
    # where out starts, 33 run into it
    at = dict(K_raw=None, V_raw=None, C_V=0x8000000, out=0x1000000 + 32 * 2 * 4096 * 32 * 2)
    for pages, status in ((32, WS), (33, ALIAS)):
        assert _call_paged(lib, _problem(raw_window=0),
                           _pages(page_rows=4096, beacon_pages=pages, raw_table=None,
                                  raw_pages=0), ptrs=at) == status
    assert _call_paged(lib, prob, _pages(reserved=1)) == SHAPE
    assert _call_paged(lib, prob, _pages(beacon_table=None)) == NULL
    assert _call_paged(lib, prob, _pages(raw_table=None)) == NULL
    assert _call_paged(lib, prob, _pages(beacon_table=0x250002)) == ALIGN
    assert _call_paged(lib, prob, _pages(beacon_table_width=0)) == SHAPE
    assert _call_paged(lib, prob, _pages(raw_pages=0)) == SHAPE
    # a segment without capacity needs no table, pools or pages
    assert _call_paged(lib, _problem(num_beacons=0), _pages(beacon_table=None, beacon_pages=0,
                                                            beacon_table_width=0),
                       ptrs=dict(U_K=None, U_V=None, C_K=None, C_V=None)) == WS
    assert _call_paged(lib, _problem(raw_window=0), _pages(raw_table=None, raw_pages=0),
                       ptrs=dict(K_raw=None, V_raw=None)) == WS
    # two pages of 64 rows for 65..128 rows
    assert _call_paged(lib, _problem(num_beacons=65), _pages()) == SHAPE
    assert _call_paged(lib, _problem(num_beacons=65), _pages(beacon_table_width=2)) == WS
    # the tables of a sequence are staged on chip: at most 4096 entries
    big = _problem(num_beacons=4096 * 64, raw_window=32)
    assert _call_paged(lib, big, _pages(beacon_table_width=4096)) == UNSUP
    assert _call_paged(lib, _problem(num_beacons=4095 * 64),
                       _pages(beacon_table_width=4095)) == WS
    # the raw pools are written with a new token (4 pages x 2 heads x 64 rows x 256 B)
    assert _call_paged(lib, prob, _pages(), ptrs=dict(k_new=0x3000000 + 4 * 32768 - 16)) == ALIAS
    assert _call_paged(lib, prob, _pages(), ptrs=dict(k_new=0x3000000 + 4 * 32768)) == WS
    assert _call_paged(lib, prob, _pages(raw_pages=5),
                       ptrs=dict(k_new=0x3000000 + 4 * 32768)) == ALIAS
    # outputs must not overlap the tables
    assert _call_paged(lib, prob, _pages(), ptrs=dict(lse=0x260000 - 4)) == ALIAS
    assert _call_paged(lib, prob, _pages(raw_table=0x6000000 + 8)) == ALIAS
    # the same flags and batch limits as the ragged call
    assert _call_paged(lib, _problem(batch=1025), _pages()) == UNSUP


def _call_chunk(lib, prob, Q, *, ptrs=None, ws_bytes=16):
    """slimkv_decode_attn_chunk with fake device addresses (every case fails
    validation before any HIP call: at the latest, the 16-byte workspace is
    too small)."""
    p = dict(q=0x100000, q_pos=0x200000, U_K=0x300000, U_V=0x400000, C_K=0x1000000,
             C_V=0x2000000, K_raw=0x3000000, V_raw=0x4000000, nb=0x210000, raw=0x220000,
             k_new=0x230000, v_new=0x240000, out=0x5000000, lse=0x6000000, ws=0x7000000)
    p.update(ptrs or {})
    v = {k: (None if x is None else ctypes.c_void_p(x)) for k, x in p.items()}
    return lib.slimkv_decode_attn_chunk(ctypes.byref(prob), Q, v["q"], v["q_pos"], v["U_K"],
                                        v["U_V"], v["C_K"], v["C_V"], v["K_raw"], v["V_raw"],
                                        v["nb"], v["raw"], v["k_new"], v["v_new"], v["out"],
                                        v["lse"], v["ws"], ws_bytes, None)


def test_chunk_checks(lib):
    prob = _problem()  # G = 4, batch 2, 8 query heads
    ws = lib.slimkv_chunk_workspace_bytes
    assert ws(ctypes.byref(prob), 4) > ws(ctypes.byref(prob), 1) > 0
    # the query rows of a KV head fill one 16-row tile; bf16 only
    assert ws(ctypes.byref(prob), 5) == 0 and "16" in lda.slimkv_last_error()
    assert ws(ctypes.byref(prob), 0) == 0
    assert ws(ctypes.byref(_problem(dtype="fp32")), 1) > 0
    assert ws(ctypes.byref(_problem(num_q_heads=2)), 16) > 0
    assert _call_chunk(lib, prob, 4) == WS
    assert _call_chunk(lib, prob, 4, ws_bytes=ws(ctypes.byref(prob), 4) - 1) == WS
    assert _call_chunk(lib, prob, 5) == UNSUP
    assert _call_chunk(lib, prob, 0) == SHAPE
    assert _call_chunk(lib, _problem(dtype="fp32"), 2) == WS
    flagged = _problem()
    flagged.flags = lda.SLIMKV_FLAG_DYNAMIC_TILES
    assert _call_chunk(lib, flagged, 2) == UNSUP
    assert _call_chunk(lib, prob, 2, ptrs=dict(v_new=None)) == NULL
    assert _call_chunk(lib, prob, 2, ptrs=dict(k_new=None, v_new=None)) == WS
    # q, k_new, v_new, out and lse carry the token axis: 3 tokens of q are
    # 3 x 2 x 8 x 128 x 2 bytes, so out may start right after, not before
    q_bytes = 3 * 2 * 8 * 128 * 2
    assert _call_chunk(lib, prob, 3, ptrs=dict(out=0x100000 + q_bytes)) == WS
    assert _call_chunk(lib, prob, 3, ptrs=dict(out=0x100000 + q_bytes - 16)) == ALIAS
    lse_bytes = 3 * 2 * 8 * 4
    assert _call_chunk(lib, prob, 3, ptrs=dict(lse=0x240000 - lse_bytes)) == WS
    assert _call_chunk(lib, prob, 3, ptrs=dict(lse=0x240000 - lse_bytes + 4)) == ALIAS
    # the raw window is written with new tokens
    assert _call_chunk(lib, prob, 2, ptrs=dict(k_new=0x3000000 + 64)) == ALIAS


def _call_chunk_paged(lib, prob, pages, Q, *, ptrs=None, ws_bytes=16):
    """slimkv_decode_attn_chunk_paged with fake device addresses (every case
    fails validation before any HIP call)."""
    p = dict(q=0x100000, q_pos=0x200000, U_K=0x300000, U_V=0x400000, C_K=0x1000000,
             C_V=0x2000000, K_raw=0x3000000, V_raw=0x4000000, nb=0x210000, raw=0x220000,
             k_new=0x230000, v_new=0x240000, out=0x5000000, lse=0x6000000, ws=0x7000000)
    p.update(ptrs or {})
    v = {k: (None if x is None else ctypes.c_void_p(x)) for k, x in p.items()}
    pg = ctypes.byref(pages) if pages is not None else None
    return lib.slimkv_decode_attn_chunk_paged(ctypes.byref(prob), pg, Q, v["q"], v["q_pos"],
                                              v["U_K"], v["U_V"], v["C_K"], v["C_V"], v["K_raw"],
                                              v["V_raw"], v["nb"], v["raw"], v["k_new"],
                                              v["v_new"], v["out"], v["lse"], v["ws"], ws_bytes,
                                              None)


def test_chunk_paged_checks(lib):
    """The paged chunk call takes the chunk call's token rules and the paged
    call's table rules; its workspace is the chunk call's."""
    prob = _problem()  # G = 4: up to 4 tokens; one page of 64 rows per segment
    ws = lib.slimkv_chunk_workspace_bytes(ctypes.byref(prob), 4)
    assert _call_chunk_paged(lib, prob, _pages(), 4) == WS
    assert _call_chunk_paged(lib, prob, _pages(), 4, ws_bytes=ws - 1) == WS
    assert _call_chunk_paged(lib, prob, _pages(), 5) == UNSUP
    assert _call_chunk_paged(lib, prob, _pages(), 0) == SHAPE
    assert _call_chunk_paged(lib, _problem(dtype="fp32"), _pages(), 2) == WS
    assert _call_chunk_paged(lib, prob, None, 2) == NULL
    assert _call_chunk_paged(lib, prob, _pages(page_rows=96), 2) == SHAPE
    assert _call_chunk_paged(lib, prob, _pages(raw_table=None), 2) == NULL
    assert _call_chunk_paged(lib, prob, _pages(raw_table_width=0), 2) == SHAPE
    assert _call_chunk_paged(lib, prob, _pages(), 2, ptrs=dict(v_new=None)) == NULL
    # the raw pool (4 pages x 2 heads x 64 rows x 128 x 2 B = 0x20000) is written
    assert _call_chunk_paged(lib, prob, _pages(), 2, ptrs=dict(k_new=0x3000000 + 0x20000)) == WS
    assert _call_chunk_paged(lib, prob, _pages(), 2,
                             ptrs=dict(k_new=0x3000000 + 0x20000 - 16)) == ALIAS
    # out carries the token axis (3 tokens: 3 x 2 x 8 x 128 x 4 bytes) and must not meet a table
    out_bytes = 3 * 2 * 8 * 128 * 4
    assert _call_chunk_paged(lib, prob, _pages(), 3, ptrs=dict(out=0x250000 - out_bytes)) == WS
    assert _call_chunk_paged(lib, prob, _pages(), 3,
                             ptrs=dict(out=0x250000 - out_bytes + 4)) == ALIAS


def test_alibi_checks(lib):
    prob = _problem()
    v = {k: ctypes.c_void_p(x) for k, x in dict(q=0x100000, q_pos=0x200000, U_K=0x300000,
                                                 U_V=0x400000, C_K=0x1000000, C_V=0x2000000,
                                                 K_raw=0x3000000, V_raw=0x4000000, sl=0x210000,
                                                 out=0x5000000, lse=0x6000000,
                                                 ws=0x7000000).items()}

    def call(sl=v["sl"], first=15, stride=16, lse=v["lse"], p=prob):
        return lib.slimkv_decode_attn_alibi(ctypes.byref(p), v["q"], v["q_pos"], v["U_K"],
                                            v["U_V"], v["C_K"], v["C_V"], v["K_raw"], v["V_raw"],
                                            sl, first, stride, v["out"], lse, v["ws"], 16, None)
    assert call() == WS  # every pointer check passes; the workspace is too small
    assert call(sl=None) == NULL and "slopes" in lda.slimkv_last_error()
    assert call(sl=ctypes.c_void_p(0x210002)) == ALIGN
    assert call(stride=-1) == SHAPE
    assert call(first=-5) == SHAPE
    assert call(first=2**31 - 100, stride=16) == SHAPE  # the last of 64 beacons overflows int32
    assert call(first=2**31 - 100, stride=0) == WS
    assert call(lse=ctypes.c_void_p(0x210000 - 16)) == ALIAS  # lse runs into the slopes (8 heads)
    assert call(lse=ctypes.c_void_p(0x210000 - 64)) == WS


def test_reconstruct_rope_checks(lib):
    prob = _problem()
    v = {k: ctypes.c_void_p(x) for k, x in dict(q=0x100000, q_pos=0x200000, U_K=0x300000,
                                                 U_V=0x400000, C_K=0x1000000, C_V=0x2000000,
                                                 K_raw=0x3000000, V_raw=0x4000000, bp=0x210000,
                                                 out=0x5000000, lse=0x6000000,
                                                 ws=0x7000000).items()}

    def call(bp=v["bp"], ws_bytes=16, out=v["out"], p=prob):
        return lib.slimkv_reconstruct_rope_attn(ctypes.byref(p), v["q"], v["q_pos"], v["U_K"],
                                                v["U_V"], v["C_K"], v["C_V"], v["K_raw"],
                                                v["V_raw"], bp, out, v["lse"], v["ws"], ws_bytes,
                                                None)
    assert call() == WS  # every pointer check passes; the workspace is too small
    assert call(bp=None) == NULL and "beacon_pos" in lda.slimkv_last_error()
    assert call(bp=ctypes.c_void_p(0x210002)) == ALIGN
    assert call(out=ctypes.c_void_p(0x210000 - 16)) == ALIAS  # out runs into beacon_pos
    assert call(bp=None, p=_problem(num_beacons=0)) == WS      # no beacons: no positions needed



def test_bench_helpers_reject_bad_arguments(lib):
    """The measurement helpers check their arguments before any HIP call."""
    vp = ctypes.c_void_p
    src, sink = vp(0x1000000), vp(0x100)
    assert lib.slimkv_bench_stream_read(None, 1024, 4, 0, sink, None) == NULL
    assert lib.slimkv_bench_stream_read(src, 1024, 4, 0, None, None) == NULL
    assert lib.slimkv_bench_stream_read(vp(0x1000008), 1024, 4, 0, sink, None) == ALIGN
    assert lib.slimkv_bench_stream_read(src, 1000, 4, 0, sink, None) == SHAPE
    assert lib.slimkv_bench_stream_read(src, 0, 4, 0, sink, None) == SHAPE
    assert lib.slimkv_bench_stream_read(src, 1 << 31, 4, 0, sink, None) == SHAPE
    assert lib.slimkv_bench_stream_read(src, 1024, 3, 0, sink, None) == UNSUP
    assert lib.slimkv_bench_stream_read(src, 1024, 4, -1, sink, None) == SHAPE
    assert lib.slimkv_bench_stream_read(src, 1024, 4, 0, vp(0x1000010), None) == ALIAS
    assert lib.slimkv_bench_flush(None, 1024, 0, None) == NULL
    assert lib.slimkv_bench_flush(vp(0x1000004), 1024, 0, None) == ALIGN
    assert lib.slimkv_bench_flush(src, 1000, 0, None) == SHAPE


def test_alibi_struct_layout():
    text = HEADER.read_text()
    body = re.search(r"typedef struct slimkv_alibi \{(.*?)\} slimkv_alibi;", text, re.S).group(1)
    names = re.findall(r"^\s*(?:const float\*|int32_t)\s+(\w+);", body, re.M)
    assert names == [f for f, _ in binding.slimkv_alibi._fields_]
    assert ctypes.sizeof(binding.slimkv_alibi) == 16


def test_alibi_serving_checks(lib):
    """The ALiBi forms of the serving calls: the rotary call's checks, plus a
    NULL alibi or slopes, beacon positions that leave int32, and misaligned
    slopes -- all before any HIP call."""
    vp = ctypes.c_void_p
    p = dict(q=0x100000, q_pos=0x200000, U_K=0x300000, U_V=0x400000, C_K=0x1000000,
             C_V=0x2000000, K_raw=0x3000000, V_raw=0x4000000, nb=0x210000, raw=0x220000,
             k_new=0x230000, v_new=0x240000, out=0x5000000, lse=0x6000000, ws=0x7000000)
    v = {k: vp(x) for k, x in p.items()}
    tail = (v["q"], v["q_pos"], v["U_K"], v["U_V"], v["C_K"], v["C_V"], v["K_raw"], v["V_raw"],
            v["nb"], v["raw"], v["k_new"], v["v_new"], v["out"], v["lse"], v["ws"], 1 << 30, None)
    prob = _problem()
    pages = lda.make_pages(page_rows=64)
    pages.beacon_table_width = 1
    pages.raw_table_width = 1
    pages.beacon_pages = pages.raw_pages = 4
    pages.beacon_table = 0x250000
    pages.raw_table = 0x260000

    def calls(al):
        a = ctypes.byref(al) if al is not None else None
        pp = ctypes.byref(prob)
        return [lib.slimkv_decode_attn_ragged_alibi(pp, a, *tail),
                lib.slimkv_decode_attn_paged_alibi(pp, ctypes.byref(pages), a, *tail),
                lib.slimkv_decode_attn_chunk_alibi(pp, a, 2, *tail),
                lib.slimkv_decode_attn_chunk_paged_alibi(pp, ctypes.byref(pages), a, 2, *tail)]

    good = binding.slimkv_alibi(0x280000, 15, 16)
    # with good parameters every call gets as far as the (too small) workspace
    ws_small = tail[:-2] + (16, None)
    pp = ctypes.byref(prob)
    assert lib.slimkv_decode_attn_ragged_alibi(pp, ctypes.byref(good), *ws_small) == WS
    assert lib.slimkv_decode_attn_chunk_alibi(pp, ctypes.byref(good), 2, *ws_small) == WS
    assert calls(None) == [NULL] * 4
    assert calls(binding.slimkv_alibi(None, 15, 16)) == [NULL] * 4
    assert calls(binding.slimkv_alibi(0x280000, -1, 16)) == [SHAPE] * 4
    assert calls(binding.slimkv_alibi(0x280000, 0, -16)) == [SHAPE] * 4
    assert calls(binding.slimkv_alibi(0x280000, 0, 1 << 30)) == [SHAPE] * 4  # 63 beacons past int32
    assert calls(binding.slimkv_alibi(0x280002, 15, 16)) == [ALIGN] * 4
    assert calls(binding.slimkv_alibi(0x5000000, 15, 16)) == [ALIAS] * 4  # slopes inside out
