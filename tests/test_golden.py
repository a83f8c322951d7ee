"""The oracle reproduces the hand-worked examples in tests/golden/ exactly."""
from __future__ import annotations

import numpy as np
import pytest

import golden_cases

CASES = golden_cases.load()


@pytest.mark.parametrize("case", CASES, ids=[c["id"] for c in CASES])
def test_oracle_matches_hand_example(case):
    got = golden_cases.run_oracle(case)
    for key, want in case["expected"].items():
        np.testing.assert_array_equal(got[key], np.asarray(want, np.float64), err_msg=key)
