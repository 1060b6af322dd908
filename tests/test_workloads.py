"""Pins of the seeded input generators (CPU only).

The expected block counts and the tiny mask were computed independently of this
module from the stated recipe (torch CPU generators; the mask readings listed in
the workloads module docstring).  If the RNG of a future torch changes them, the
recipe must be re-derived, not these numbers edited to match."""
import numpy as np
import pytest
import torch

import workloads as W

NNZ = {"tiny_f32": 25, "dense_bf16": 16384, "causal_bf16": 133120,
       "sparse_bf16": 24647, "long_bf16": 107572}
ROW_COUNTS = {"tiny_f32": (2, 4), "dense_bf16": (16, 16), "causal_bf16": (1, 64),
              "sparse_bf16": (3, 23), "long_bf16": (1, 55)}


@pytest.mark.parametrize("name", W.ORDER)
def test_mask_block_counts(name):
    w = W.WORKLOADS[name]
    m = W.make_mask(w)
    assert tuple(m.shape) == (w.B, w.H, w.n_q, w.n_k) and m.dtype == torch.uint8
    assert int(m.sum()) == NNZ[name]
    c = m.sum(-1)
    assert (int(c.min()), int(c.max())) == ROW_COUNTS[name]


def test_tiny_mask_values():
    m = W.make_mask(W.WORKLOADS["tiny_f32"])
    assert m[0, 0].tolist() == [[1, 0, 1, 1], [1, 1, 1, 0], [1, 0, 1, 1], [1, 1, 1, 1]]
    assert m[0, 1].tolist() == [[1, 0, 1, 1], [0, 1, 1, 0], [1, 0, 1, 1], [1, 1, 1, 1]]


def test_mask_structure():
    w = W.WORKLOADS["sparse_bf16"]
    m = W.make_mask(w)[0]
    i = torch.arange(w.n_q)
    for d in range(4):  # window of 4 ending at the diagonal
        j = (i - d).clamp(min=0)
        assert bool(m[:, i, j].all())
    assert bool(m[:, :, :2].all())  # global key blocks
    w = W.WORKLOADS["long_bf16"]
    m = W.make_mask(w)[0]
    assert not bool(torch.triu(m.to(torch.int32), diagonal=1).any())  # causal
    assert bool(m[:, torch.arange(w.n_q), torch.arange(w.n_q)].all())  # diagonal
    ii, jj = torch.meshgrid(torch.arange(w.n_q), torch.arange(w.n_k), indexing="ij")
    assert bool(m[:, (jj % 16 == 0) & (jj <= ii)].all())  # strided


def test_qkv_recipe():
    q, k, v = W.make_qkv(1, 2, 64, 8, torch.bfloat16, seed=0)
    g = torch.Generator().manual_seed(0)
    q32 = torch.randn(1, 2, 64, 8, generator=g)
    assert torch.equal(q, q32.to(torch.bfloat16))
    assert q.dtype == k.dtype == v.dtype == torch.bfloat16
    assert not torch.equal(q, k) and not torch.equal(k, v)


def test_scale_and_flops():
    assert W.WORKLOADS["dense_bf16"].scale == float(np.float32(1 / np.sqrt(128)))
    w = W.WORKLOADS["dense_bf16"]
    assert W.flops(W.make_mask(w), 128, 128, 128) == 4 * 128 * 16384 * 128 * 128


def test_sample_rows_in_range():
    w = W.WORKLOADS["causal_bf16"]
    rows = W.sample_rows(w.B, w.H, w.S, w.block_q, 40, mask=W.make_mask(w))
    assert len(rows) >= 40 and rows.min() >= 0 and rows.max() < w.B * w.H * w.S
    assert len(np.unique(rows)) == len(rows)


def test_token_causal_elem_workload():
    """The element-level token-causal workload keeps exactly the lower triangle:
    S (S + 1) / 2 elements per head, and its expanded mask is tril (checked on a
    small copy of the same recipe)."""
    from brute import expand_elem
    w = W.ELEM_WORKLOADS["causal_elem_bf16"]
    st, pidx, pbits = W.make_elem_mask(w)
    assert W.kept_elements(st, pidx, pbits, w.block_q, w.block_k) == w.B * w.H * w.S * (w.S + 1) // 2
    small = W.Workload("t", 1, 1, 512, 64, 128, 128, "bf16", "token_causal")
    s2, p2, b2 = W.make_elem_mask(small)
    full = expand_elem(s2.numpy(), p2.numpy(), b2.numpy().view(np.uint32), 128, 128)
    assert np.array_equal(full[0, 0], np.tril(np.ones((512, 512), dtype=bool)))
