"""Plant plausible mistakes in the oracle (on the CPU, via -DORACLE_MUTANT=n)
and check that the pin suite catches every one of them:
 1 causal off-by-one (a row misses its own key)
 2 ancestors' visible prefixes dropped (fork offset ignored)
 3 wrong GQA grouping (h % Hkv instead of contiguous groups)
 4 decay not applied to the erase term of Eq. 4
 5 state used transposed in Eq. 4
 6 softmax scale dropped
 7 output read from the state before the update (S_{t-1} q_t)
 8 positions off by one below a fork
 9 conv: rows before the segment's own first row not read (window lost at a fork)
10 conv: predecessors taken one row too far back
11 sliding window one key too wide (t_x - t_y <= W)
12 two-way rule misses the last row of the own segment
13 projection: the last term of the sum dropped
14 projection: the index buffer of rows ignored
"""
import pytest

import oracle
from tests import pins


@pytest.mark.parametrize("mutant", range(1, 15))
def test_mutant_is_caught(mutant):
    path = oracle.build(force=False, extra_flags=(f"-DORACLE_MUTANT={mutant}",))
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(libpath=path)
        except (AssertionError, oracle.OracleError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {mutant} passed every pin"
