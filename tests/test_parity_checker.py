"""The parity checker itself (CPU only): given the oracle's own results as a
stand-in for the GPU's, it passes; a planted NaN head, a planted output error
or a tiles_used far from any threshold must fail it."""
import numpy as np
import pytest

import art_inputs as A
from tests.gpu_util import check_parity
from tests.helpers import run_oracle


@pytest.fixture(scope="module")
def case_and_oracle():
    c = A.config(3, small=True, seed=1, batch=2, ctx=1024)
    return c, run_oracle(c)


def test_oracle_results_pass(case_and_oracle):
    c, ora = case_and_oracle
    r = check_parity(c, ora.out.copy(), ora.tiles_used.copy(), ora=ora)
    assert r["max_abs"] == 0.0 and r["near"] == []


def test_nan_head_fails(case_and_oracle):
    c, ora = case_and_oracle
    out = ora.out.copy()
    out[1, 5] = np.nan  # one head, the others exact
    with pytest.raises(AssertionError, match="non-finite"):
        check_parity(c, out, ora.tiles_used.copy(), ora=ora)


def test_output_error_fails(case_and_oracle):
    c, ora = case_and_oracle
    out = ora.out.copy()
    out[0, 2, 7] += 3e-3  # above the 2e-3 bar of bf16 caches
    with pytest.raises(AssertionError, match="max"):
        check_parity(c, out, ora.tiles_used.copy(), ora=ora)


def test_tiles_used_far_from_threshold_fails(case_and_oracle):
    c, ora = case_and_oracle
    used = ora.tiles_used.copy()
    used[0, 0] = used[0, 0] + 3 if used[0, 0] + 3 <= 16 else used[0, 0] - 3
    with pytest.raises(AssertionError, match="away from the thresholds"):
        check_parity(c, ora.out.copy(), used, ora=ora)
