"""Shared helpers of the GPU tests: library loading, tolerance checks against the
fp64 oracle, and input staging."""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import block_sparse_flash_mask_amd as bs  # noqa: E402

# Tolerances of the forward output against the fp64 oracle run on the same
# (already rounded) input values.
TOL = {
    "f32": dict(out_max=1e-4, out_mean=1e-4, lse=1e-5),
    "bf16": dict(out_max=1e-2, out_mean=1e-3, lse=1e-3),
}


def ensure_built():
    if not os.path.exists(bs.LIB_PATH):
        from block_sparse_flash_mask_amd import build
        build.build()
    return bs.library()


def say(*a):
    print(*a, flush=True)


def dkey(t):
    return "f32" if t.dtype == torch.float32 else "bf16"


def to_dev(*ts):
    return [t.cuda() for t in ts]


def compare(out_gpu, lse_gpu, out_ref, lse_ref, kind, what=""):
    """Check GPU (out, lse) against the oracle's (out_ref, lse_ref) float64 arrays of
    the same leading shape.  Returns the error stats."""
    out = out_gpu.detach().float().cpu().double().numpy().reshape(out_ref.shape)
    lse = lse_gpu.detach().float().cpu().double().numpy().reshape(lse_ref.shape)
    assert not np.isnan(out).any(), (what, "NaN in out")
    assert not np.isnan(lse).any(), (what, "NaN in lse")
    empty = np.isneginf(lse_ref)
    assert np.all(np.isneginf(lse[empty])), (what, "empty rows must have lse == -inf")
    assert np.all(out[empty] == 0.0), (what, "empty rows must have out == 0")
    assert np.all(np.isfinite(lse[~empty])), (what, "non-empty rows need a finite lse")
    err = np.abs(out - out_ref)
    stats = dict(out_max=float(err.max()) if err.size else 0.0,
                 out_mean=float(err.mean()) if err.size else 0.0,
                 lse=float(np.abs(lse[~empty] - lse_ref[~empty]).max()) if (~empty).any() else 0.0)
    tol = TOL[kind]
    assert stats["out_max"] <= tol["out_max"], (what, stats)
    assert stats["out_mean"] <= tol["out_mean"], (what, stats)
    assert stats["lse"] <= tol["lse"], (what, stats)
    return stats


def rand_qkv(B, H, S, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, S, D, generator=g)
    k = torch.randn(B, H, S, D, generator=g)
    v = torch.randn(B, H, S, D, generator=g)
    return q.to(dtype), k.to(dtype), v.to(dtype)


def rand_mask(B, H, n_q, n_k, p, seed, diag=True, empty_rows=()):
    g = torch.Generator().manual_seed(seed)
    m = torch.rand(B, H, n_q, n_k, generator=g) < p
    if diag:
        i = torch.arange(min(n_q, n_k))
        m[:, :, i, i] = True
    m = m.to(torch.uint8)
    for (b, h, i) in empty_rows:
        m[b, h, i] = 0
    return m
