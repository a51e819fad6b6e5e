"""The oracle reproduces the hand-derived cases under ``tests/golden/``."""
import numpy as np
import pytest

import oracle
from golden_cases import all_cases
from oracle_refs import round_to, widen

CASES = all_cases()


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_case(case):
    dt = case["dtype"]
    x = round_to(case["x"], dt)
    assert np.array_equal(widen(x, dt), case["x"]), "fixture value not exact in its type"
    D = x.size
    L = case["slice"][1] - case["slice"][0]
    c = round_to(case["cos"], dt).reshape(1, 1, 1, L)
    s = round_to(case["sin"], dt).reshape(1, 1, 1, L)
    y = x.reshape(1, 1, 1, D).copy()
    oracle.rope_rows(y, (1, 1, 1, D), dt, c, s, case["mode"], case["slice"], case["direction"])
    assert widen(y, dt).ravel().tolist() == case["expect"].tolist()


def test_all_fixtures_present():
    assert len(CASES) >= 7
