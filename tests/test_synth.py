"""The seeded input generator: determinism, shapes, the rank draw, and the
shared token stream between a compressed cache's raw window and the full
cache."""

import hashlib

import numpy as np
import pytest
import torch

import synth


def _digest(inp: synth.LayerInputs) -> str:
    h = hashlib.sha256()
    for name in ("q", "q_pos", "U_K", "U_V", "C_K", "C_V", "K_raw", "V_raw"):
        h.update(synth.to_numpy_storage(getattr(inp, name)).tobytes())
    return h.hexdigest()


def test_layer_is_deterministic_and_seed_dependent():
    wl = synth.get_workload("c1")
    a = _digest(synth.make_layer(wl, 0))
    assert a == _digest(synth.make_layer(wl, 0))
    assert a != _digest(synth.make_layer(wl, 0, base_seed=1))


@pytest.mark.parametrize("key", ["c1", "c2"])
def test_shapes_and_dtypes(key):
    wl = synth.get_workload(key)
    inp = synth.make_layer(wl, 0)
    B, Hq, Hkv, d, r = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.ranks[0]
    dt = torch.float32 if wl.dtype == "fp32" else torch.bfloat16
    assert inp.q.shape == (B, Hq, d) and inp.q.dtype == dt
    assert inp.q_pos.dtype == torch.int32 and int(inp.q_pos[0]) == wl.context - 1
    assert inp.U_K.shape == (Hkv, d, r) and inp.U_V.shape == (Hkv, d, r)
    assert inp.C_K.shape == (B, Hkv, wl.num_beacons, r) and inp.C_V.dtype == dt
    assert inp.K_raw.shape == (B, Hkv, wl.raw_window, d)
    for t in (inp.q, inp.C_K, inp.K_raw):
        assert t.is_contiguous()


def test_value_scale_follows_sigma():
    wl = synth.get_workload("c2")  # sigma 0.5
    inp = synth.make_layer(wl, 0)
    std = inp.C_K.float().std().item()
    assert abs(std - 0.5) < 0.01


def test_bases_have_orthonormal_columns():
    u = synth.orthonormal_basis(128, 48, seed=5)
    assert torch.allclose(u.T @ u, torch.eye(48, dtype=torch.float64), atol=1e-12)
    g = torch.Generator().manual_seed(5)
    a = torch.randn((128, 48), generator=g, dtype=torch.float64)
    assert (torch.diagonal(u.T @ a) > 0).all()  # sign convention: diag(R) > 0


@pytest.mark.parametrize("layers,mean", [(32, 64), (48, 64)])
def test_rank_draw_meets_budget(layers, mean):
    for seed in range(300):
        ranks = synth.draw_ranks(layers, mean, seed)
        assert len(ranks) == layers and sum(ranks) == layers * mean
        assert set(ranks) <= set(synth.RANK_SET)


def test_workload_ranks_budget():
    assert sum(synth.get_workload("c3").ranks) == 32 * 64
    assert sum(synth.get_workload("c4").ranks) == 48 * 64


def test_raw_window_is_tail_of_full_cache():
    wl = synth.get_workload("c1")
    inp = synth.make_layer(wl, 0)
    k, v = synth.make_full_kv(wl, 0)
    assert k.shape[2] == wl.context
    assert torch.equal(k[:, :, -wl.raw_window:], inp.K_raw)
    assert torch.equal(v[:, :, -wl.raw_window:], inp.V_raw)


def test_unit_slices_layout():
    wl = synth.get_workload("c2")
    inp = synth.make_layer(wl, 0, num_beacons=32, raw_window=16)
    u = synth.unit_slices(inp, 3, 5)
    assert u["q"].shape == (1, 4, 128) and u["q"].dtype == np.uint16
    full_q = synth.to_numpy_storage(inp.q)
    assert np.array_equal(u["q"][0], full_q[3, 20:24])
    assert u["C_K"].shape == (1, 1, 32, 64)
