"""Mask compaction on the GPU must equal the oracle's CSR bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import bs, ensure_built, say

pytestmark = pytest.mark.gpu


def _check(mask):
    ensure_built()
    B, H, n_q, n_k = mask.shape
    say("compact", tuple(mask.shape), int(mask.sum()))
    rp, ci = bs.compact_mask(mask.cuda())
    torch.cuda.synchronize()
    rp = rp.cpu().numpy()
    orp, oci = oracle.compact(mask)
    assert np.array_equal(rp, orp)
    nnz = int(orp[-1])
    assert np.array_equal(ci.cpu().numpy()[:nnz], oci)


@pytest.mark.parametrize("name", W.ORDER)
def test_compact_workloads(name):
    _check(W.make_mask(W.WORKLOADS[name]))


@pytest.mark.parametrize("shape,p,seed", [
    ((1, 1, 1, 1), 1.0, 0),
    ((2, 3, 4, 4), 0.0, 1),       # all zero
    ((1, 2, 8, 8), 1.0, 2),       # all one
    ((2, 2, 5, 70), 0.3, 3),      # n_k not a multiple of 64
    ((1, 3, 7, 129), 0.05, 4),
    ((1, 1, 9, 512), 0.5, 5),
    ((3, 5, 11, 64), 0.5, 6),
    ((1, 1, 5000, 3), 0.5, 7),    # more rows than one scan tile
])
def test_compact_random(shape, p, seed):
    g = torch.Generator().manual_seed(seed)
    m = (torch.rand(*shape, generator=g) < p).to(torch.uint8)
    _check(m)


def test_compact_single_column():
    m = torch.zeros(2, 2, 6, 40, dtype=torch.uint8)
    m[..., 17] = 1
    _check(m)


def test_compact_nonbinary_bytes():
    g = torch.Generator().manual_seed(9)
    m = torch.randint(0, 256, (1, 2, 6, 100), generator=g, dtype=torch.uint8)
    m[m < 128] = 0
    _check(m)
