"""Dense NumPy fp64 brute force of masked softmax attention, for tiny shapes only.

It takes the literal route the pages print for the masking step ("Writing Pallas
Kernels for JAX", section "Writing the Kernel Logic: Load, Compute, Store"): build
the full S x S score matrix, expand the block mask to element level, set masked
scores to -inf, softmax over the whole row, multiply by V.  The row softmax and
log-sum-exp come from scipy.special (a library routine), so this shares no
arithmetic with the oracle's two-pass loop.  A row whose scores are all -inf is
given out = 0, lse = -inf (the empty-row convention).
"""
import numpy as np
from scipy.special import logsumexp


def widen(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def expand_mask(mask, block_q, block_k):
    m = widen(mask) != 0  # [B,H,nq,nk]
    return np.repeat(np.repeat(m, block_q, axis=2), block_k, axis=3)  # [B,H,S,S]


def brute_fwd(q, k, v, mask, block_q, block_k, scale):
    q, k, v = widen(q), widen(k), widen(v)
    scale = float(np.float32(scale))
    full = expand_mask(mask, block_q, block_k)
    s = scale * np.matmul(q, np.swapaxes(k, -1, -2))
    s = np.where(full, s, -np.inf)
    with np.errstate(invalid="ignore", divide="ignore"):
        lse = logsumexp(s, axis=-1)
        p = np.exp(s - lse[..., None])
    empty = ~full.any(axis=-1)
    p[empty] = 0.0
    lse[empty] = -np.inf
    return np.matmul(p, v), lse, p


def brute_compact(mask):
    m = widen(mask) != 0
    rows = m.reshape(-1, m.shape[-1])
    row_ptr = [0]
    cols = []
    for r in rows:
        nz = np.nonzero(r)[0]
        cols.extend(int(c) for c in nz)
        row_ptr.append(len(cols))
    return np.array(row_ptr, dtype=np.int32), np.array(cols, dtype=np.int32)
