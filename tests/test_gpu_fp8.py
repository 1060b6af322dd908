"""fp8 forward on the GPU (bsattn_fwd_fp8) against the fp64 oracle on the same
e4m3 inputs (the oracle widens each e4m3 byte exactly).

Tolerance, per element, derived from the arithmetic: e4m3 x e4m3 products are
exact in fp32 and the scores are fp32 sums of D of them; the row max,
exponentials, row sums and lse stay fp32.  The softmax weights P (stored relative
to a reference maximum m_ref <= the row maximum M, so P <= 2^8) are rounded to
e4m3 before P V: a relative error <= 2^-4 for P >= 2^-6 and an absolute error
<= 2^-10 below (subnormal spacing 2^-9).  Divided by the row sum (>= the sum of
2^(s_j - M) = 1 / w_max), the error of weight j is <= 2^-4 w_j + 2^-10 w_max, so
  |out - ref| <= sum_j (2^-4 w_j + 2^-10 w_max) |v_j| + 2^-9 |ref| (bf16 out)
                 + D 2^-24 sum_j w_j |v_j| (fp32 sums),
held with a factor 2; the mean error must stay below half the mean bound.
lse: fp32 scores and sums, |error| <= 2e-4."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import bs, ensure_built, rand_mask, say

pytestmark = pytest.mark.gpu


def _fp8_inputs(B, H, S, D, seed):
    g = torch.Generator().manual_seed(seed)
    return [torch.randn(B, H, S, D, generator=g).to(torch.float8_e4m3fn) for _ in range(3)]


def _bound_rows(q, k, v, mask, bq, bk, scale, rows, ref):
    """Per-element bounds [len(rows), D] for flat query rows (numpy, fp64)."""
    B, H, S, D = q.shape
    qf, kf, vf = (t.to(torch.float64).reshape(B * H, S, D).numpy() for t in (q, k, v))
    m = mask.numpy().reshape(B * H, S // bq, S // bk) != 0
    out = np.zeros((len(rows), D))
    for i, r in enumerate(rows):
        bh, s = divmod(int(r), S)
        keys = np.repeat(m[bh, s // bq], bk)
        if not keys.any():
            continue
        sc = float(np.float32(scale)) * (kf[bh][keys] @ qf[bh, s])
        w = np.exp(sc - sc.max())
        w /= w.sum()
        av = np.abs(vf[bh][keys])
        out[i] = (2.0 ** -4 * (w @ av) + 2.0 ** -10 * w.max() * av.sum(0) + D * 2.0 ** -24 * (w @ av))
    return 2 * (out + 2.0 ** -9 * np.abs(ref))


def _bound_dense_full(q, k, v, scale, ref):
    """The bounds of _bound_rows for an all-ones mask over every row, one head at a
    time as matrix products (numpy, fp64)."""
    B, H, S, D = q.shape
    qf, kf, vf = (t.to(torch.float64).reshape(B * H, S, D).numpy() for t in (q, k, v))
    out = np.empty((B * H, S, D))
    for bh in range(B * H):
        sc = float(np.float32(scale)) * (qf[bh] @ kf[bh].T)
        w = np.exp(sc - sc.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        av = np.abs(vf[bh])
        wav = w @ av
        out[bh] = 2.0 ** -4 * wav + 2.0 ** -10 * w.max(axis=1, keepdims=True) * av.sum(0) + D * 2.0 ** -24 * wav
    return 2 * (out.reshape(ref.shape) + 2.0 ** -9 * np.abs(ref))


def _check(out, lse, ro, rl, bound, what):
    o = out.float().cpu().double().numpy().reshape(ro.shape)
    l = lse.cpu().double().numpy().reshape(rl.shape)
    empty = np.isneginf(rl)
    assert np.all(np.isneginf(l[empty])) and np.all(o[empty] == 0), (what, "empty rows")
    assert np.all(np.isfinite(o)), (what, "non-finite out")
    err = np.abs(o - ro)
    bad = err > bound + 1e-30
    assert not bad.any(), (what, int(bad.sum()), float((err - bound).max()))
    assert err.mean() <= 0.5 * bound.mean(), (what, float(err.mean()), float(bound.mean()))
    el = float(np.abs(l[~empty] - rl[~empty]).max()) if (~empty).any() else 0.0
    assert el <= 2e-4, (what, "lse", el)
    return float(err.max()), el


def _run(B, H, S, D, bq, bk, scale, seed, p=0.5, what=""):
    ensure_built()
    q, k, v = _fp8_inputs(B, H, S, D, seed)
    mask = rand_mask(B, H, S // bq, S // bk, p, seed, empty_rows=[(0, 0, 1)])
    say("fwd_fp8", what, (B, H, S, D), (bq, bk), scale)
    out, lse = bs.fwd_fp8(q.cuda(), k.cuda(), v.cuda(), mask.cuda(), bq, bk, scale)
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(q, k, v, mask, bq, bk, scale)
    rows = np.arange(B * H * S)
    bound = _bound_rows(q, k, v, mask, bq, bk, scale, rows, ro.reshape(-1, D)).reshape(ro.shape)
    say("  max err", _check(out, lse, ro, rl, bound, what))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("blocks", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_fp8_small(D, blocks):
    bq, bk = blocks
    _run(1, 2, 512, D, bq, bk, 1.0 / np.sqrt(D), 3 + D + bk, what="%s" % (blocks,))


def test_fp8_negative_scale_dense_mask():
    _run(2, 1, 384, 128, 128, 64, -0.2, 17, p=1.1, what="negative scale, all blocks")


def test_fp8_planned_matches_and_empty_mask():
    """plan + fwd_fp8_planned equals fwd_fp8 bit for bit; an all-zero mask gives
    out = 0, lse = -inf."""
    ensure_built()
    B, H, S, D, b = 1, 2, 512, 128, 128
    q, k, v = (t.cuda() for t in _fp8_inputs(B, H, S, D, 23))
    mask = rand_mask(B, H, S // b, S // b, 0.5, 23).cuda()
    o1, l1 = bs.fwd_fp8(q, k, v, mask, b, b)
    ws = torch.empty(bs.fp8_workspace_size(B, H, S, D, b, b), dtype=torch.uint8, device="cuda")
    bs.plan(mask, S, b, b, workspace=ws)
    o2, l2 = bs.fwd_fp8_planned(q, k, v, ws, b, b)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    z = torch.zeros_like(mask)
    o3, l3 = bs.fwd_fp8(q, k, v, z, b, b)
    torch.cuda.synchronize()
    assert torch.all(o3 == 0) and torch.all(torch.isneginf(l3))


def test_fp8_workload_dense_sampled():
    """The dense shape (B4 H16 S2048 D128, 128x128 blocks) in fp8 at full size on
    sampled rows."""
    w = W.WORKLOADS["dense_bf16"]
    ensure_built()
    q, k, v = _fp8_inputs(w.B, w.H, w.S, w.D, 0)
    mask = torch.ones(w.B, w.H, w.n_q, w.n_k, dtype=torch.uint8)
    say("fwd_fp8 workload", tuple(q.shape))
    out, lse = bs.fwd_fp8(q.cuda(), k.cuda(), v.cuda(), mask.cuda(), w.block_q, w.block_k, w.scale)
    torch.cuda.synchronize()
    rows = W.sample_rows(w.B, w.H, w.S, w.block_q, 48)
    ro, rl = oracle.fwd_rows(q, k, v, mask, w.block_q, w.block_k, w.scale, rows)
    go = out.reshape(-1, w.D)[torch.as_tensor(rows, device=out.device)]
    gl = lse.reshape(-1)[torch.as_tensor(rows, device=lse.device)]
    bound = _bound_rows(q, k, v, mask, w.block_q, w.block_k, w.scale, rows, ro)
    say("  max err", _check(go, gl, ro, rl, bound, "dense fp8"))


def test_fp8_workload_dense_full():
    """The dense shape (B4 H16 S2048 D128, 128x128 blocks) in fp8 at full size, every
    output element against its bound."""
    w = W.WORKLOADS["dense_bf16"]
    ensure_built()
    q, k, v = _fp8_inputs(w.B, w.H, w.S, w.D, 0)
    mask = torch.ones(w.B, w.H, w.n_q, w.n_k, dtype=torch.uint8)
    say("fwd_fp8 workload, full output", tuple(q.shape))
    out, lse = bs.fwd_fp8(q.cuda(), k.cuda(), v.cuda(), mask.cuda(), w.block_q, w.block_k, w.scale)
    torch.cuda.synchronize()
    # The oracle gets the e4m3 values widened to fp32 (exact; its own e4m3 decoding
    # is pinned byte for byte to the same conversion) so that its inner loop skips
    # the per-element decode: identical output, about six times sooner.
    say("oracle, full output on", oracle.max_threads(), "threads ...")
    ro, rl = oracle.fwd(q.float(), k.float(), v.float(), mask, w.block_q, w.block_k, w.scale)
    bound = _bound_dense_full(q, k, v, w.scale, ro)
    say("  max err", _check(out, lse, ro, rl, bound, "dense fp8, full output"))
