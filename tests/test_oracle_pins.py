"""The CPU oracle against its pins (see tests/pins.py for what each pin rests on)."""
import pytest

import oracle
from tests import pins


@pytest.fixture(scope="module")
def O():
    return oracle.Oracle()


@pytest.mark.parametrize("pin", pins.ALL, ids=[p.__name__ for p in pins.ALL])
def test_pin(O, pin):
    pin(O)


def test_rejects_empty_sequence(O):
    import workloads as W
    inp = pins._tiny([3, 4, 5], 1)
    args = list(W.oracle_args(inp))
    args[6] = args[6].copy()
    args[6][1] = 0
    with pytest.raises(ValueError):
        O.decode(*args)


def test_sampled_pairs_match_full(O):
    import numpy as np
    import workloads as W
    inp = pins._tiny([20, 50, 9], 5)
    full, lse = O.decode(*W.oracle_args(inp))
    pairs = [(2, 1), (0, 0), (1, 1)]
    out, l2 = O.decode(*W.oracle_args(inp), pairs=pairs)
    for i, (b, h) in enumerate(pairs):
        assert np.array_equal(out[i], full[b, h]) and l2[i] == lse[b, h]
