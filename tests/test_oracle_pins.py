"""The fp64 oracle against its pins (closed forms, limits, invariants, worked examples)."""
import pytest

import _pins


@pytest.mark.parametrize("check", _pins.ALL_CHECKS, ids=lambda c: getattr(c, "__name__", "check"))
def test_oracle_pin(orc, check):
    check(orc)


def test_oracle_threads_invariant(orc):
    """Channel-parallel execution does not change any bit of the result."""
    import numpy as np
    rng = np.random.default_rng(42)
    x, delta, A, B, C, D = _pins.random_case(rng, 2, 30, 17, 16)
    y1, h1 = orc.scan(x, delta, A, B, C, D, threads=1)
    y4, h4 = orc.scan(x, delta, A, B, C, D, threads=4)
    assert np.array_equal(y1, y4) and np.array_equal(h1, h4)


def test_oracle_empty_sequence(orc):
    """L = 0: no outputs, and the final state is the initial state."""
    import numpy as np
    x = np.zeros((2, 0, 3))
    h0 = np.arange(2 * 3 * 4, dtype=np.float64).reshape(2, 3, 4)
    y, hf = orc.scan(x, x, -np.ones((3, 4)), np.zeros((2, 0, 4)), np.zeros((2, 0, 4)), np.ones(3), h0=h0)
    assert y.shape == (2, 0, 3)
    assert np.array_equal(hf, h0)
