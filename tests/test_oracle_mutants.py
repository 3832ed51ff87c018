"""Each planted mistake in the oracle (ORACLE_MUTANT=k) must fail at least one pin.

The mistakes are the plausible ones for this method: a dropped RoPE term, a transposed W_UK,
the wrong softmax scale, the page table ignored, the last token dropped, the wrong head's
W_UV, a missing log in the log-sum-exp, the wrong head's RoPE query, and in the page gather
a zero fill that starts one row late or rows copied without their RoPE part.
"""
import os
import tempfile

import pytest

import oracle
from oracle import build as obuild
from tests import pins

MUTANTS = {1: "rope dropped", 2: "W_UK transposed", 3: "scale 1/sqrt(d_n)",
           4: "page table ignored", 5: "last token dropped", 6: "W_UV of head 0",
           7: "lse without log", 8: "q_rope of head 0", 9: "gather zero fill one row late",
           10: "gather drops k_R"}


@pytest.mark.parametrize("k", sorted(MUTANTS), ids=[MUTANTS[k] for k in sorted(MUTANTS)])
def test_mutant_is_caught(k):
    with tempfile.TemporaryDirectory() as d:
        path = obuild.build(out=os.path.join(d, "libmut%d.so" % k), mutant=k)
        O = oracle.Oracle(path=path)
        assert O.mutant == k
        caught = []
        for pin in pins.ALL:
            try:
                pin(O)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(pin.__name__)
        assert caught, "mutant %d (%s) passed every pin" % (k, MUTANTS[k])
