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


def expand_elem(states, pidx, pbits, block_q, block_k):
    """Element mask [B,H,S,S] of block states (0 empty, 1 full, else partial) with
    bit tiles pbits[n_tiles][block_q][block_k / 32] (bit c % 32 of word c / 32 of
    row i keeps element (i, c) of a partial block using that tile)."""
    st = np.asarray(widen(states), dtype=np.int64)
    pi = np.asarray(widen(pidx), dtype=np.int64)
    pb = np.ascontiguousarray(np.asarray(pbits).astype(np.uint32))
    B, H, nq, nk = st.shape
    if pb.shape[0]:
        tiles = np.unpackbits(pb.view(np.uint8).reshape(pb.shape[0], block_q, -1), axis=-1,
                              bitorder="little").astype(bool)
    full = np.zeros((B, H, nq * block_q, nk * block_k), dtype=bool)
    for b in range(B):
        for h in range(H):
            for i in range(nq):
                for j in range(nk):
                    blk = full[b, h, i * block_q:(i + 1) * block_q, j * block_k:(j + 1) * block_k]
                    if st[b, h, i, j] == 1:
                        blk[:] = True
                    elif st[b, h, i, j] > 1:
                        blk[:] = tiles[pi[b, h, i, j]]
    return full


def brute_fwd(q, k, v, mask, block_q, block_k, scale):
    return brute_fwd_full(q, k, v, expand_mask(mask, block_q, block_k), scale)


def brute_fwd_full(q, k, v, full, scale):
    """The same with an element mask full [B,H,S,S] (True = kept)."""
    q, k, v = widen(q), widen(k), widen(v)
    scale = float(np.float32(scale))
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
