"""Where the bias corrections 1 - beta^t (formed on the host in binary64 and
rounded once to binary32) become exactly 1.0f for the GPU tests' hyper-
parameters: the step ranges of tests/test_gpu_unit_bc.py fall on both sides
of each threshold (CPU only; the oracle's per-call scalars)."""
import numpy as np

import oracle
from tests.test_gpu_unit_bc import HP, RANGES


def _unit(hp, t):
    return tuple(bool(x == np.float32(1.0)) for x in oracle.scalars(hp, t)[2:4])


def test_thresholds_are_where_the_ranges_put_them():
    hp = oracle.hparams(**HP)
    assert _unit(hp, 164) == (False, False) and _unit(hp, 165) == (True, False)
    assert _unit(hp, 337) == (True, False) and _unit(hp, 338) == (True, True)
    assert all(_unit(hp, t) == (False, False) for t in RANGES["none"])
    assert all(_unit(hp, t) == (True, False) for t in RANGES["bc1"])
    assert all(_unit(hp, t) == (True, True) for t in RANGES["both"])
    assert _unit(hp, min(RANGES["bc1_switch"])) == (False, False)
    assert _unit(hp, max(RANGES["bc1_switch"])) == (True, False)
    assert _unit(hp, min(RANGES["bc2_switch"])) == (True, False)
    assert _unit(hp, max(RANGES["bc2_switch"])) == (True, True)


def test_threshold_matches_the_rounding_rule():
    """1 - x rounds to 1.0f exactly when x <= 2^-25 (the half-ulp of 1.0 from
    below is 2^-25; a tie rounds to the even 1.0f): the first t with
    beta^t <= 2^-25, computed here in binary64, is the first unit step (beta =
    0.5 meets the tie exactly at t = 25)."""
    for beta in (0.5, 0.9, 0.95, 0.99, 0.999):
        hp = oracle.hparams(beta1=beta, beta2=beta)
        b = float(np.float32(beta))
        t = 1
        while b ** t > 2.0 ** -25:
            t += 1
        assert _unit(hp, t) == (True, True), beta
        assert _unit(hp, t - 1) == (False, False), beta
