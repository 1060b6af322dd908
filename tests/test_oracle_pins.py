"""The fp64 oracle pinned against brute force, library special cases, closed
forms and invariants (CPU only).  See oracle_checks.py for what pins what."""
import pytest

import oracle
import oracle_checks as C


@pytest.mark.parametrize("check", C.ALL, ids=[f.__name__ for f in C.ALL])
def test_oracle_pin(check):
    check(oracle)


def test_thread_count_is_per_call():
    """An explicit thread count applies to that call only, and the result does not
    depend on it (each row is computed by one thread in a fixed order)."""
    import torch
    g = torch.Generator().manual_seed(1)
    q, k, v = (torch.randn(1, 2, 128, 32, generator=g, dtype=torch.float64) for _ in range(3))
    mask = torch.ones(1, 2, 2, 2, dtype=torch.uint8)
    n0 = oracle.max_threads()
    o1, l1 = oracle.fwd(q, k, v, mask, 64, 64, 0.2, nthreads=1)
    assert oracle.max_threads() == n0
    o2, l2 = oracle.fwd(q, k, v, mask, 64, 64, 0.2)
    assert (o1 == o2).all() and (l1 == l2).all()
