"""The oracle rejects malformed rounds (reading: live segments hold >= 1
contiguous token; a root forks at 0; a fork lies within its parent; cached
histories sit above live segments and are continued from their end)."""
import pytest

import oracle
from tests.malformed import CASES, arrays


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_oracle_rejects(case):
    ts, par, fk, cl, kind = arrays(case)
    with pytest.raises(oracle.OracleError) as e:
        oracle.index(ts, par, fk, cl)
    assert e.value.kind == kind
