"""Each planted mistake in the oracle (built with HS2REF_MUTANT=n) must fail at
least one pin: evidence that the pins would catch such a slip in the oracle."""
import numpy as np
import pytest

import oracle
from tests import pins

MUTANTS = {
    1: "softmax scale dropped",
    2: "wrong GQA head-to-group mapping",
    3: "current token dropped from the causal range",
    4: "scores from unnormalised weights",
    5: "ties broken toward the higher position",
    6: "window excludes the current token",
    9: "sparse layer reads the neighbouring head's query",
    10: "bridge weight read transposed",
    11: "E4M3FN exponent bias 8",
    12: "LSE without the log",
    13: "block mass by max instead of sum",
    14: "top-k takes k+1",
    15: "full-layer output sums keys instead of values",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: f"m{m}")
def test_mutant_is_caught(mutant):
    oracle.build(mutant)
    failures = []
    with np.errstate(all="ignore"):
        for pin in pins.ALL_PINS:
            try:
                pin(mutant)
            except (AssertionError, RuntimeError, ValueError, IndexError) as e:
                failures.append(f"{pin.__name__}: {str(e)[:80]}")
    assert failures, f"no pin caught mutant {mutant} ({MUTANTS[mutant]})"


# Planted mistakes in the oracle's Python layer (the FP8 cache write).
PY_MUTANTS = {
    21: "old rows re-encoded with the scale ratio inverted",
    22: "scale grown without re-encoding the old rows",
    23: "new scale without the division by 448",
}


@pytest.mark.parametrize("mutant", sorted(PY_MUTANTS), ids=lambda m: f"m{m}")
def test_python_mutant_is_caught(mutant):
    failures = []
    with np.errstate(all="ignore"):
        for pin in (pins.pin_fp8_write_keep_vs_torch, pins.pin_fp8_write_grow_doubling,
                    pins.pin_fp8_write_grow_nearest):
            try:
                pin(mutant)
            except (AssertionError, RuntimeError, ValueError, IndexError) as e:
                failures.append(f"{pin.__name__}: {str(e)[:80]}")
    assert failures, f"no pin caught mutant {mutant} ({PY_MUTANTS[mutant]})"
