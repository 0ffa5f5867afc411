"""The oracle against its stored regression fixtures (tests/golden/*.json,
written by tests/golden/make_golden.py from tiny seeded inputs).  The pages
print no worked example of the attention, so these fixtures pin the
oracle to its own reviewed outputs: a change to its arithmetic fails here
until the fixtures are regenerated on purpose."""

import importlib.util
import json
import pathlib

import numpy as np
import pytest

GOLDEN = pathlib.Path(__file__).resolve().parent / "golden"
_spec = importlib.util.spec_from_file_location("make_golden", GOLDEN / "make_golden.py")
make_golden = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(make_golden)


@pytest.mark.parametrize("name", sorted(make_golden.CASES))
def test_oracle_reproduces_fixture(name):
    doc = json.loads((GOLDEN / f"{name}.json").read_text())
    entry, params, _ = make_golden.CASES[name]
    assert doc["entry"] == entry and doc["params"] == params, "fixture and case list disagree"
    got = make_golden.run_case(name)
    assert sorted(got) == sorted(doc["values"])
    for key, vals in doc["values"].items():
        exp = np.asarray(vals, dtype=np.float64).reshape(doc["shapes"][key])
        assert got[key].shape == exp.shape, key
        # -inf (a row with nothing to attend) must match exactly
        assert np.array_equal(np.isneginf(got[key]), np.isneginf(exp)), key
        fin = np.isfinite(exp)
        np.testing.assert_allclose(got[key][fin], exp[fin], rtol=1e-13, atol=1e-15, err_msg=key)
