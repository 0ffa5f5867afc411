"""Seeded tensor generator for one layer of a decode-attention workload.

Layouts (row-major, contiguous), with G = H_q / H_kv and r the layer rank:
    q       [B, H_q, d]          decode query, before RoPE
    q_pos   [B]       int32      absolute position of the decode query
    U_K     [H_kv, d, r]         beacon key basis (orthonormal columns)
    U_V     [H_kv, d, r]         beacon value basis (orthonormal columns)
    C_K     [B, H_kv, N_b, r]    latent beacon keys (carry no rotation)
    C_V     [B, H_kv, N_b, r]    latent beacon values
    K_raw   [B, H_kv, W, d]      raw-window keys, already rotated at their positions
    V_raw   [B, H_kv, W, d]      raw-window values

Distributions.  Every tensor except the bases is i.i.d. N(0, sigma^2),
drawn in fp32 and rounded once to the storage dtype (round-to-nearest-even
for bf16).  Raw keys are drawn directly in their rotated form: a rotation
of each (i, i + d/2) pair maps an isotropic Gaussian pair to another one,
so rotated i.i.d. Gaussian keys are distributed exactly like unrotated
ones, and the generator needs no positional arithmetic.  The bases are
the Q factor of a seeded N(0,1) d x r matrix (fp64 QR, columns signed so
that diag(R) > 0), rounded to the storage dtype.

Token rows (raw keys and values, and a full uncompressed cache) are drawn in
blocks of ``TOKEN_BLOCK`` positions with one seed per block, so the raw
window of a compressed cache is bit-identical to the last rows of the full
cache of the same workload and layer.

Seeds: each tensor's seed is derived from (base seed, workload index,
layer, tensor id, extra) through numpy's SeedSequence, then fed to a torch
generator on the target device.  Values generated on the CPU and on a GPU
therefore differ, but each is reproducible on its own device.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

from .configs import Workload

TOKEN_BLOCK = 128

_IDS = {"q": 1, "U_K": 2, "U_V": 3, "C_K": 4, "C_V": 5, "K_tok": 6, "V_tok": 7, "lengths": 8,
        "k_new": 9, "v_new": 10, "pages": 11}

_TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16}


def _seed(base: int, wl: Workload, layer: int, name: str, *extra: int) -> int:
    ss = np.random.SeedSequence([base, wl.index, layer, _IDS[name], *extra])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _gauss(shape, seed: int, sigma: float, dtype: str, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(_TORCH_DTYPE[dtype])


def orthonormal_basis(d: int, r: int, seed: int) -> torch.Tensor:
    """Q factor (d x r, fp64, CPU) of a seeded Gaussian matrix, diag(R) > 0."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    a = torch.randn((d, r), generator=g, dtype=torch.float64)
    qm, rm = torch.linalg.qr(a)
    signs = torch.sign(torch.diagonal(rm))
    signs[signs == 0] = 1.0
    return qm * signs


def _tokens(wl: Workload, layer: int, name: str, base: int, first: int, count: int, device):
    """Rows [first, first + count) of the token cache ``name`` ([B,H_kv,count,d])."""
    assert first % TOKEN_BLOCK == 0 and count % TOKEN_BLOCK == 0
    blocks = []
    for start in range(first, first + count, TOKEN_BLOCK):
        blk = start // TOKEN_BLOCK
        blocks.append(
            _gauss((wl.batch, wl.num_kv_heads, TOKEN_BLOCK, wl.head_dim),
                   _seed(base, wl, layer, name, blk), wl.sigma, wl.dtype, device))
    if not blocks:
        return torch.empty((wl.batch, wl.num_kv_heads, 0, wl.head_dim),
                           dtype=_TORCH_DTYPE[wl.dtype], device=device)
    return torch.cat(blocks, dim=2).contiguous()


@dataclasses.dataclass
class LayerInputs:
    """All tensors of one layer call, on one device."""

    workload: Workload
    layer: int
    rank_k: int
    rank_v: int
    q: torch.Tensor
    q_pos: torch.Tensor
    U_K: torch.Tensor
    U_V: torch.Tensor
    C_K: torch.Tensor
    C_V: torch.Tensor
    K_raw: torch.Tensor
    V_raw: torch.Tensor

    @property
    def num_beacons(self) -> int:
        return int(self.C_K.shape[2])

    @property
    def raw_window(self) -> int:
        return int(self.K_raw.shape[2])

    def to(self, device) -> "LayerInputs":
        moved = {f.name: getattr(self, f.name) for f in dataclasses.fields(self)}
        for k, v in moved.items():
            if isinstance(v, torch.Tensor):
                moved[k] = v.to(device)
        return LayerInputs(**moved)


def make_layer(wl: Workload, layer: int = 0, *, base_seed: int = 0, device="cpu",
               num_beacons: int | None = None, raw_window: int | None = None,
               rank_v: int | None = None) -> LayerInputs:
    """Generate one layer of ``wl`` on ``device``.

    ``num_beacons`` / ``raw_window`` override the workload's values (tests
    use this for ragged and degenerate shapes); ``rank_v`` gives the value
    latents a rank other than the key latents'.  Raw rows always end at the
    decode position: they cover positions [T - W, T).
    """
    nb = wl.num_beacons if num_beacons is None else num_beacons
    w = wl.raw_window if raw_window is None else raw_window
    r = wl.ranks[layer]
    rv = r if rank_v is None else rank_v
    d = wl.head_dim
    dt = _TORCH_DTYPE[wl.dtype]

    q = _gauss((wl.batch, wl.num_q_heads, d), _seed(base_seed, wl, layer, "q"), wl.sigma,
               wl.dtype, device)
    q_pos = torch.full((wl.batch,), wl.q_pos, dtype=torch.int32, device=device)
    uk = torch.stack([orthonormal_basis(d, r, _seed(base_seed, wl, layer, "U_K", h, r))
                      for h in range(wl.num_kv_heads)]).to(dt).to(device)
    uv = torch.stack([orthonormal_basis(d, rv, _seed(base_seed, wl, layer, "U_V", h, rv))
                      for h in range(wl.num_kv_heads)]).to(dt).to(device)
    ck = _gauss((wl.batch, wl.num_kv_heads, nb, r), _seed(base_seed, wl, layer, "C_K", nb, r),
                wl.sigma, wl.dtype, device)
    cv = _gauss((wl.batch, wl.num_kv_heads, nb, rv), _seed(base_seed, wl, layer, "C_V", nb, rv),
                wl.sigma, wl.dtype, device)
    if w % TOKEN_BLOCK == 0 and wl.context % TOKEN_BLOCK == 0:
        kr = _tokens(wl, layer, "K_tok", base_seed, wl.context - w, w, device)
        vr = _tokens(wl, layer, "V_tok", base_seed, wl.context - w, w, device)
    else:  # ragged windows (tests): one block, seeded by the window length
        shape = (wl.batch, wl.num_kv_heads, w, d)
        kr = _gauss(shape, _seed(base_seed, wl, layer, "K_tok", 1 << 30, w), wl.sigma, wl.dtype,
                    device)
        vr = _gauss(shape, _seed(base_seed, wl, layer, "V_tok", 1 << 30, w), wl.sigma, wl.dtype,
                    device)
    return LayerInputs(wl, layer, r, rv, q, q_pos, uk, uv, ck, cv, kr, vr)


def make_full_kv(wl: Workload, layer: int = 0, *, base_seed: int = 0, device="cpu"):
    """Uncompressed cache of all T tokens, [B, H_kv, T, d] each (keys rotated)."""
    k = _tokens(wl, layer, "K_tok", base_seed, 0, wl.context, device)
    v = _tokens(wl, layer, "V_tok", base_seed, 0, wl.context, device)
    return k, v


@dataclasses.dataclass
class StepInputs:
    """What a serving decode step adds to a layer's cache arrays: each
    sequence's live beacon and raw rows, and the step's new token (its key
    before rotation, and its value) per KV head."""

    num_beacons: torch.Tensor  # [B] int32
    raw_len: torch.Tensor      # [B] int32
    k_new: torch.Tensor        # [B, H_kv, d]
    v_new: torch.Tensor        # [B, H_kv, d]

    def to(self, device) -> "StepInputs":
        return StepInputs(*(getattr(self, f.name).to(device) for f in dataclasses.fields(self)))


def make_step(wl: Workload, inp: LayerInputs, *, base_seed: int = 0, device="cpu",
              beacons=(0.0, 1.0), raw=(0.0, 1.0), fixed: dict | None = None) -> StepInputs:
    """Seeded per-sequence lengths for ``inp``'s capacity-sized arrays and
    the step's new token.  Live rows are drawn uniformly from
    [lo * capacity, hi * capacity] for the given fractions (beacons, raw);
    ``fixed`` maps a sequence index to a (beacons, raw) pair that overrides
    its draw (edge cases: empty, full, beyond the capacity)."""
    ncap, wcap = inp.num_beacons, inp.raw_window
    ss = np.random.SeedSequence([base_seed, wl.index, inp.layer, _IDS["lengths"], ncap, wcap])
    rng = np.random.default_rng(ss)
    nb = rng.integers(int(beacons[0] * ncap), int(beacons[1] * ncap) + 1, size=wl.batch)
    rw = rng.integers(int(raw[0] * wcap), int(raw[1] * wcap) + 1, size=wl.batch)
    for b, (x, y) in (fixed or {}).items():
        nb[b], rw[b] = x, y
    shape = (wl.batch, wl.num_kv_heads, wl.head_dim)
    k = _gauss(shape, _seed(base_seed, wl, inp.layer, "k_new"), wl.sigma, wl.dtype, device)
    v = _gauss(shape, _seed(base_seed, wl, inp.layer, "v_new"), wl.sigma, wl.dtype, device)
    return StepInputs(torch.from_numpy(nb.astype(np.int32)).to(device),
                      torch.from_numpy(rw.astype(np.int32)).to(device), k, v)


@dataclasses.dataclass
class ChunkInputs:
    """A chunk of Q query tokens per sequence: the queries (token t of
    sequence b at position q_pos[b] + t), each sequence's live rows, and the
    chunk's tokens (keys before rotation, values) per KV head."""

    q: torch.Tensor            # [B, Q, H_q, d]
    num_beacons: torch.Tensor  # [B] int32
    raw_len: torch.Tensor      # [B] int32
    k_new: torch.Tensor        # [B, Q, H_kv, d]
    v_new: torch.Tensor        # [B, Q, H_kv, d]

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[1])

    def to(self, device) -> "ChunkInputs":
        return ChunkInputs(*(getattr(self, f.name).to(device) for f in dataclasses.fields(self)))


def make_chunk(wl: Workload, inp: LayerInputs, num_tokens: int, *, base_seed: int = 0,
               device="cpu", beacons=(0.0, 1.0), raw=(0.0, 1.0),
               fixed: dict | None = None) -> ChunkInputs:
    """Seeded chunk of ``num_tokens`` query tokens per sequence for ``inp``'s
    capacity-sized arrays: queries and tokens N(0, sigma^2) in the storage
    dtype, lengths drawn as in ``make_step``."""
    step = make_step(wl, inp, base_seed=base_seed, device=device, beacons=beacons, raw=raw,
                     fixed=fixed)
    B, Q, d = wl.batch, num_tokens, wl.head_dim
    q = _gauss((B, Q, wl.num_q_heads, d), _seed(base_seed, wl, inp.layer, "q", Q), wl.sigma,
               wl.dtype, device)
    shape = (B, Q, wl.num_kv_heads, d)
    k = _gauss(shape, _seed(base_seed, wl, inp.layer, "k_new", Q), wl.sigma, wl.dtype, device)
    v = _gauss(shape, _seed(base_seed, wl, inp.layer, "v_new", Q), wl.sigma, wl.dtype, device)
    return ChunkInputs(q, step.num_beacons, step.raw_len, k, v)


@dataclasses.dataclass
class PagedCache:
    """A layer's cache laid out in pages drawn from shared pools:
    C_K, C_V [beacon_pages, H_kv, page_rows, r] and K_raw, V_raw
    [raw_pages, H_kv, page_rows, d]; sequence b's row i of a segment lies in
    page table[b, i // page_rows] at row i % page_rows."""

    page_rows: int
    C_K: torch.Tensor
    C_V: torch.Tensor
    K_raw: torch.Tensor
    V_raw: torch.Tensor
    beacon_table: torch.Tensor  # [B, width] int32
    raw_table: torch.Tensor     # [B, width] int32

    @property
    def beacon_pages(self) -> int:
        return int(self.C_K.shape[0])

    @property
    def raw_pages(self) -> int:
        return int(self.K_raw.shape[0])


def _nan_fill(t: torch.Tensor) -> torch.Tensor:
    return t.fill_(float("nan"))


def _page_out(x: torch.Tensor, live: torch.Tensor, table: torch.Tensor, pages: int,
              page_rows: int) -> torch.Tensor:
    """Scatter capacity rows x [B, H, cap, w] into a pool of ``pages`` pages
    through ``table``; rows at or past each sequence's ``live`` count, and
    pages no sequence maps, hold NaN."""
    B, H, cap, w = x.shape
    n = table.shape[1]
    pool = _nan_fill(torch.empty((pages, H, page_rows, w), dtype=x.dtype, device=x.device))
    if cap == 0 or n == 0:
        return pool
    padded = _nan_fill(torch.empty((B, H, n * page_rows, w), dtype=x.dtype, device=x.device))
    rows = torch.arange(cap, device=x.device)
    keep = (rows[None, :] < live[:, None].to(x.device)).view(B, 1, cap, 1)
    padded[:, :, :cap] = torch.where(keep, x, torch.full_like(x, float("nan")))
    blocks = padded.view(B, H, n, page_rows, w).permute(0, 2, 1, 3, 4).reshape(B * n, H,
                                                                                 page_rows, w)
    pool[table.reshape(-1).to(torch.int64).to(x.device)] = blocks
    return pool


def make_paged(inp: LayerInputs, step: StepInputs, *, page_rows: int, base_seed: int = 0,
               spare: int = 3, extra_width: int = 1) -> PagedCache:
    """Page out ``inp``'s capacity arrays: each sequence gets
    ceil(capacity / page_rows) pages per segment, at page ids drawn as a
    seeded permutation of a pool with ``spare`` more pages than needed.
    Rows past a sequence's live length (lengths clamped to the capacity,
    as the kernels clamp them) and unmapped pages hold NaN, so reading any
    of them would show.  Tables get ``extra_width`` more columns, set to -1."""
    wl = inp.workload
    B = wl.batch
    ncap, wcap = inp.num_beacons, inp.raw_window
    nbp, nrp = -(-ncap // page_rows), -(-wcap // page_rows)
    ss = np.random.SeedSequence([base_seed, wl.index, inp.layer, _IDS["pages"], page_rows])
    rng = np.random.default_rng(ss)

    def table(need):
        pages = B * need + (spare if need else 0)
        ids = rng.permutation(pages)[:B * need].reshape(B, need).astype(np.int32)
        full = np.full((B, need + extra_width if need else 0), -1, dtype=np.int32)
        full[:, :need] = ids
        return pages, torch.from_numpy(full).to(inp.q.device)

    bpages, bt = table(nbp)
    rpages, rt = table(nrp)
    nb_live = step.num_beacons.clamp(0, ncap)
    w_live = step.raw_len.clamp(0, wcap)
    return PagedCache(
        page_rows,
        _page_out(inp.C_K, nb_live, bt[:, :nbp], bpages, page_rows),
        _page_out(inp.C_V, nb_live, bt[:, :nbp], bpages, page_rows),
        _page_out(inp.K_raw, w_live, rt[:, :nrp], rpages, page_rows),
        _page_out(inp.V_raw, w_live, rt[:, :nrp], rpages, page_rows),
        bt, rt)


def alibi_slopes(num_heads: int) -> np.ndarray:
    """Per-head ALiBi slopes (inputs of the ALiBi variant): for n heads, n a
    power of two, the geometric sequence 2^(-8/n), 2^(-16/n), ...; otherwise
    the slopes of the largest power of two below n, then every other slope
    of twice as many heads."""
    def pow2(n):
        start = 2.0 ** (-8.0 / n)
        return [start ** (i + 1) for i in range(n)]
    n = 1 << (num_heads.bit_length() - 1)
    s = pow2(n)
    if n < num_heads:
        s += pow2(2 * n)[0::2][:num_heads - n]
    return np.asarray(s, dtype=np.float64)


def beacon_grid(ratio: int) -> tuple:
    """Positions of beacons that each summarise `ratio` tokens, beacon j
    covering tokens [j * ratio, (j + 1) * ratio) and placed at its last
    token: (first, stride) = (ratio - 1, ratio)."""
    return ratio - 1, ratio


def to_numpy_storage(t: torch.Tensor) -> np.ndarray:
    """CPU numpy view of a tensor in its storage format (bf16 as uint16 bits)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def unit_slices(inp: LayerInputs, b: int, h: int) -> dict:
    """Storage-format numpy arrays of one (b, kv head) unit, shaped as a
    problem with batch 1 and a single KV head (G query heads)."""
    g = inp.workload.group
    return {
        "q": to_numpy_storage(inp.q[b:b + 1, h * g:(h + 1) * g]),
        "q_pos": to_numpy_storage(inp.q_pos[b:b + 1]),
        "U_K": to_numpy_storage(inp.U_K[h:h + 1]),
        "U_V": to_numpy_storage(inp.U_V[h:h + 1]),
        "C_K": to_numpy_storage(inp.C_K[b:b + 1, h:h + 1]),
        "C_V": to_numpy_storage(inp.C_V[b:b + 1, h:h + 1]),
        "K_raw": to_numpy_storage(inp.K_raw[b:b + 1, h:h + 1]),
        "V_raw": to_numpy_storage(inp.V_raw[b:b + 1, h:h + 1]),
    }
