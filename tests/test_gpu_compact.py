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


def _rnd(x):
    return (x + 255) // 256 * 256


def _unsnake(a):
    """Undo the dispatch layout: every other complete group of four is reversed."""
    a = a.copy()
    n = len(a)
    for g0 in range(4, n - 3, 8):
        a[g0:g0 + 4] = a[g0:g0 + 4][::-1].copy()
    return a


def _check_plan(mask, block_q=128, block_k=128, mask_dev=None):
    """bsattn_plan's three arrays: counts and lists equal the oracle's compaction
    bit for bit; each XCD chunk of the order holds exactly its own rows, then -1
    padding, head by head with each head's rows by non-increasing count (or by
    non-increasing count alone when a chunk spans too many head x count bins),
    laid out with every other complete group of four reversed."""
    ensure_built()
    B, H, n_q, n_k = mask.shape
    S = n_q * block_q
    assert n_k * block_k == S
    say("plan", tuple(mask.shape), int(mask.sum()))
    ws = bs.plan(mask.cuda() if mask_dev is None else mask_dev, S, block_q, block_k)
    torch.cuda.synchronize()
    w = ws.cpu().numpy().view(np.int32)
    R = B * H * n_q
    counts = w[:R]
    lists = w[_rnd(4 * R) // 4:][:R * n_k].reshape(R, n_k)
    chunk = (R + 7) // 8
    order = w[(_rnd(4 * R) + _rnd(4 * R * n_k)) // 4:][:8 * chunk]
    hq = (n_q + 1) // 2
    P = B * H * hq
    pchunk = (P + 7) // 8
    porder = w[(_rnd(4 * R) + _rnd(4 * R * n_k) + _rnd(4 * 8 * chunk)) // 4:][:8 * pchunk]
    orp, oci = oracle.compact(mask)
    assert np.array_equal(counts, np.diff(orp))
    # pair order: each chunk holds its own pairs, by head, then by the longer list
    cnt_r = np.diff(orp)
    for x in range(8):
        p0, p1 = min(x * pchunk, P), min((x + 1) * pchunk, P)
        got = porder[x * pchunk:(x + 1) * pchunk]
        npr = p1 - p0
        assert np.array_equal(np.sort(got[:npr]), np.arange(p0, p1)), ("pairs", x)
        assert np.all(got[npr:] == -1), ("pairs", x)
        pr = _unsnake(got[:npr])
        bh, j = pr // hq, pr % hq
        ra = bh * n_q + 2 * j
        cb = np.where(2 * j + 1 < n_q, cnt_r[np.minimum(ra + 1, R - 1)], 0)
        c = np.maximum(cnt_r[ra], cb)
        if ((pchunk + hq - 1) // hq + 1) * (n_k + 1) <= 4096:
            assert np.all(bh[:-1] <= bh[1:]), ("pairs", x)
            same = bh[:-1] == bh[1:]
            assert np.all(c[:-1][same] >= c[1:][same]), ("pairs", x)
        else:
            assert np.all(c[:-1] >= c[1:]), ("pairs", x)
    for i in range(R):
        assert np.array_equal(lists[i, :counts[i]], oci[orp[i]:orp[i + 1]]), i
    for x in range(8):
        r0, r1 = min(x * chunk, R), min((x + 1) * chunk, R)
        got = order[x * chunk:(x + 1) * chunk]
        nr = r1 - r0
        assert np.array_equal(np.sort(got[:nr]), np.arange(r0, r1)), x
        assert np.all(got[nr:] == -1), x
        rows = _unsnake(got[:nr])
        c = counts[rows]
        by_head = ((chunk + n_q - 1) // n_q + 1) * (n_k + 1) <= 4096
        if by_head:
            hd = rows // n_q
            assert np.all(hd[:-1] <= hd[1:]), x
            same = hd[:-1] == hd[1:]
            assert np.all(c[:-1][same] >= c[1:][same]), x
        else:
            assert np.all(c[:-1] >= c[1:]), x


@pytest.mark.parametrize("name", W.ORDER)
def test_plan_workloads(name):
    w = W.WORKLOADS[name]
    _check_plan(W.make_mask(w), w.block_q, w.block_k)


@pytest.mark.parametrize("shape,p,seed", [
    ((1, 1, 1, 1), 1.0, 0),        # one row: seven empty chunks
    ((1, 1, 5, 5), 0.5, 1),        # fewer rows than XCDs
    ((2, 3, 7, 7), 0.3, 2),        # R = 42, a ragged last chunk
    ((1, 2, 40, 40), 0.0, 3),      # all empty
    ((1, 4, 64, 64), 1.0, 4),      # all full: every count ties
    ((3, 5, 33, 33), 0.2, 5),
    ((2, 3, 20, 20), 0.4, 11),     # rows of 20 bytes: 4-byte mask loads
    # a mask over 4 MiB: the row lists and the orders come from two launches
    ((1, 8, 1024, 1024), 0.02, 8),
])
def test_plan_random(shape, p, seed):
    g = torch.Generator().manual_seed(seed)
    m = (torch.rand(*shape, generator=g) < p).to(torch.uint8)
    _check_plan(m)


def test_plan_order_without_heads():
    """A chunk spanning 65 heads x 65 counts (> 4096 bins) is sorted by count alone."""
    g = torch.Generator().manual_seed(6)
    m = (torch.rand(4, 128, 128, 64, generator=g) < 0.1).to(torch.uint8)
    _check_plan(m, 64, 128)


def test_plan_large_chunks():
    """More than 8192 rows per XCD chunk (131072 rows): the two-launch plan."""
    g = torch.Generator().manual_seed(10)
    m = (torch.rand(4, 128, 256, 128, generator=g) < 0.05).to(torch.uint8)
    _check_plan(m, 64, 128)


def test_plan_unaligned_mask():
    """A mask tensor starting at an odd address: the counts are read byte by byte."""
    g = torch.Generator().manual_seed(12)
    m = (torch.rand(2, 3, 32, 32, generator=g) < 0.3).to(torch.uint8)
    big = torch.zeros(m.numel() + 1, dtype=torch.uint8, device="cuda")
    view = big[1:].view(m.shape)
    view.copy_(m.cuda())
    assert view.data_ptr() % 2 == 1
    _check_plan(m, mask_dev=view)
