"""The fp64 oracle against independent references, invariants and closed
forms (see tests/oracle_pins.py for what each pin states)."""

import numpy as np
import pytest

import oracle
from oracle_pins import ALL_PINS, random_problem, run_oracle


@pytest.fixture(scope="module")
def library():
    return oracle.build()


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, library):
    pin(library)


def test_storage_widening_is_exact(library):
    """bf16 bits and fp32 inputs give exactly the result of their fp64 widening."""
    p = random_problem(21, B=2, Hkv=2, G=4, d=128, nb=11, rk=32, rv=32, w=7)
    for name in ("q", "U_K", "U_V", "C_K", "C_V", "K_raw", "V_raw"):
        p[name] = p[name].astype(np.float32)
    out32, lse32 = run_oracle(p, library)
    wide = {k: (v.astype(np.float64) if isinstance(v, np.ndarray) and v.dtype == np.float32 else v)
            for k, v in p.items()}
    out64, lse64 = run_oracle(wide, library)
    assert np.array_equal(out32, out64) and np.array_equal(lse32, lse64)
    bits = {k: (v.view(np.uint32) >> 16).astype(np.uint16)
            if isinstance(v, np.ndarray) and v.dtype == np.float32 else v for k, v in p.items()}
    outb, lseb = run_oracle(bits, library)
    widened = {k: (oracle.bf16_to_f64(v) if isinstance(v, np.ndarray) and v.dtype == np.uint16
                   else v) for k, v in bits.items()}
    outw, lsew = run_oracle(widened, library)
    assert np.array_equal(outb, outw) and np.array_equal(lseb, lsew)


def test_unit_subset_matches_full(library):
    p = random_problem(22, B=3, Hkv=2, G=2, d=16, nb=5, rk=4, rv=4, w=3)
    full, full_lse = run_oracle(p, library)
    sub, sub_lse = oracle.decode(p["q"], p["q_pos"], p["U_K"], p["U_V"], p["C_K"], p["C_V"],
                                 p["K_raw"], p["V_raw"], num_kv_heads=2, scale=p["scale"],
                                 rope_theta=p["theta"], units=[(2, 1), (0, 0)], library=library)
    for b, h in [(2, 1), (0, 0)]:
        assert np.array_equal(sub[b, 2 * h:2 * h + 2], full[b, 2 * h:2 * h + 2])
        assert np.array_equal(sub_lse[b, 2 * h:2 * h + 2], full_lse[b, 2 * h:2 * h + 2])
    assert np.isnan(sub[1]).all()


def test_weights_sum_to_one_under_large_scores(library):
    """Scores in the thousands: the softmax stays finite and normalised."""
    d = 16
    p = random_problem(23, B=1, Hkv=1, G=2, d=d, nb=6, rk=d, rv=d, w=4)
    p["U_K"] = np.eye(d)[None]
    p["U_V"] = np.eye(d)[None]
    cv = np.zeros_like(p["C_V"])
    cv[..., 3] = 1.0
    vr = np.zeros_like(p["V_raw"])
    vr[..., 3] = 1.0
    out, lse = run_oracle(p, library, q=p["q"] * 3000.0, C_V=cv, V_raw=vr)
    assert np.all(np.isfinite(lse))
    assert np.allclose(out[..., 3], 1.0, atol=1e-13, rtol=0)


def test_rejects_bad_problems(library):
    p = random_problem(24, B=1, Hkv=2, G=2, d=16, nb=2, rk=4, rv=4, w=1)
    with pytest.raises(ValueError):
        oracle.decode(p["q"][:, :3], p["q_pos"], p["U_K"], p["U_V"], p["C_K"], p["C_V"],
                      p["K_raw"], p["V_raw"], num_kv_heads=2, scale=1.0, rope_theta=1e4,
                      library=library)
    with pytest.raises(ValueError):
        oracle.decode(p["q"], p["q_pos"], p["U_K"], p["U_V"], None, None, None, None,
                      num_kv_heads=2, scale=1.0, rope_theta=1e4, library=library)
