"""The fp64 oracle pinned against brute force, library special cases, closed
forms and invariants (CPU only).  See oracle_checks.py for what pins what."""
import pytest

import oracle
import oracle_checks as C


@pytest.mark.parametrize("check", C.ALL, ids=[f.__name__ for f in C.ALL])
def test_oracle_pin(check):
    check(oracle)
