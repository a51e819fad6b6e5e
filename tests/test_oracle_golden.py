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
    tt = case["table_dtype"]
    c = round_to(case["cos"], tt).reshape(1, 1, 1, L)
    s = round_to(case["sin"], tt).reshape(1, 1, 1, L)
    assert np.array_equal(widen(c, tt).ravel(), case["cos"]), "table value not exact in its type"
    y = x.reshape(1, 1, 1, D).copy()
    oracle.rope_rows(y, (1, 1, 1, D), dt, c, s, case["mode"], case["slice"], case["direction"], table_dtype=tt)
    assert widen(y, dt).ravel().tolist() == case["expect"].tolist()


def test_all_fixtures_present():
    assert len(CASES) >= 7
