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


# ---- element-level masks ---------------------------------------------------------

def _keep_rows(st, pidx, pbits, bq, bk, rows, S):
    """Kept keys [len(rows), S] (bool) of flat query rows under an element mask:
    state 0 drops the block, 1 keeps it, anything else keeps the bits of tile
    pidx (clamped into the tile range) for the row's place in its block."""
    B, H, n_q, n_k = st.shape
    stn = st.numpy().reshape(B * H, n_q, n_k)
    pin = pidx.numpy().reshape(B * H, n_q, n_k)
    words = pbits.numpy().view(np.uint32)
    tiles = np.unpackbits(words.view(np.uint8).reshape(words.shape[0], bq, -1), axis=-1,
                          bitorder="little").astype(bool)  # [n_tiles, bq, bk]
    keep = np.zeros((len(rows), S), dtype=bool)
    for i, r in enumerate(rows):
        bh, s = divmod(int(r), S)
        qi, qr = divmod(s, bq)
        for kj in range(n_k):
            state = stn[bh, qi, kj]
            if state == 1:
                keep[i, kj * bk:(kj + 1) * bk] = True
            elif state > 1:
                t = min(max(int(pin[bh, qi, kj]), 0), tiles.shape[0] - 1)
                keep[i, kj * bk:(kj + 1) * bk] = tiles[t, qr]
    return keep


def _bound_keep(q, k, v, keep, scale, rows, ref):
    """The bound of _bound_rows for rows whose kept keys are given element by
    element (keep [len(rows), S]); rows that keep nothing get bound 0."""
    B, H, S, D = q.shape
    qf, kf, vf = (t.to(torch.float64).reshape(B * H, S, D).numpy() for t in (q, k, v))
    out = np.zeros((len(rows), D))
    for i, r in enumerate(rows):
        bh, s = divmod(int(r), S)
        keys = keep[i]
        if not keys.any():
            continue
        sc = float(np.float32(scale)) * (kf[bh][keys] @ qf[bh, s])
        w = np.exp(sc - sc.max())
        w /= w.sum()
        av = np.abs(vf[bh][keys])
        out[i] = (2.0 ** -4 * (w @ av) + 2.0 ** -10 * w.max() * av.sum(0) + D * 2.0 ** -24 * (w @ av))
    return 2 * (out + 2.0 ** -9 * np.abs(ref))


def _rand_elem(B, H, S, bq, bk, n_tiles, seed):
    """Random states (empty / full / partial), tiles per block and bit tiles; tile 0
    has an all-clear row and tile 1 is all clear, so some rows keep nothing."""
    g = np.random.default_rng(seed)
    st = g.choice(3, size=(B, H, S // bq, S // bk), p=(0.3, 0.3, 0.4)).astype(np.uint8)
    st[st == 2] = g.choice([2, 3, 200], size=int((st == 2).sum()))
    pidx = g.integers(0, n_tiles, size=st.shape).astype(np.int32)
    bits = g.random((n_tiles, bq, bk)) < 0.5
    bits[0, 3, :] = False
    bits[1] = False
    return torch.from_numpy(st), torch.from_numpy(pidx), W.pack_tiles(bits)


def _run_elem(q, k, v, st, pidx, pbits, bq, bk, scale, what):
    ensure_built()
    B, H, S, D = q.shape
    say("fwd_fp8_elem", what, (B, H, S, D), (bq, bk), scale)
    out, lse = bs.fwd_fp8_elem(q.cuda(), k.cuda(), v.cuda(), st.cuda(), pidx.cuda(), pbits.cuda(), bq, bk, scale)
    torch.cuda.synchronize()
    ro, rl = oracle.fwd_elem(q, k, v, st, pidx, pbits, bq, bk, scale)
    rows = np.arange(B * H * S)
    keep = _keep_rows(st, pidx, pbits, bq, bk, rows, S)
    bound = _bound_keep(q, k, v, keep, scale, rows, ro.reshape(-1, D)).reshape(ro.shape)
    say("  max err", _check(out, lse, ro, rl, bound, what))
    return out, lse


def test_fp8_elem_bound_helpers_match_block_form():
    """(CPU-side check of the test's own helpers, run with the GPU tests) An element
    mask whose states are only empty or full gives the kept keys and bounds of the
    block-mask form."""
    B, H, S, D, bq, bk = 1, 2, 256, 64, 64, 128
    q, k, v = _fp8_inputs(B, H, S, D, 9)
    mask = rand_mask(B, H, S // bq, S // bk, 0.5, 9)
    st = mask.clone()
    pidx = torch.zeros_like(st, dtype=torch.int32)
    pbits = W.pack_tiles(np.ones((1, bq, bk), dtype=bool))
    rows = np.arange(B * H * S)
    keep = _keep_rows(st, pidx, pbits, bq, bk, rows, S)
    m = mask.numpy().reshape(B * H, S // bq, S // bk) != 0
    want = np.stack([np.repeat(m[r // S, (r % S) // bq], bk) for r in rows])
    assert np.array_equal(keep, want)
    ref = np.random.default_rng(0).standard_normal((len(rows), D))
    assert np.allclose(_bound_keep(q, k, v, keep, 0.125, rows, ref),
                       _bound_rows(q, k, v, mask, bq, bk, 0.125, rows, ref), rtol=1e-12, atol=0)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("blocks", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_fp8_elem_small(D, blocks):
    bq, bk = blocks
    q, k, v = _fp8_inputs(1, 2, 512, D, 41 + D + bk)
    st, pidx, pbits = _rand_elem(1, 2, 512, bq, bk, 3, 5 * bq + bk + D)
    _run_elem(q, k, v, st, pidx, pbits, bq, bk, 1.0 / np.sqrt(D), "%s" % (blocks,))


@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_fp8_elem_degenerate_scales(scale):
    """A negative scale, and a zero scale (every kept score equal: a uniform
    softmax over the kept keys, no NaN from the dropped ones)."""
    q, k, v = _fp8_inputs(1, 2, 384, 128, 77)
    st, pidx, pbits = _rand_elem(1, 2, 384, 128, 64, 3, 78)
    _run_elem(q, k, v, st, pidx, pbits, 128, 64, scale, "scale %g" % scale)


def test_fp8_elem_token_causal():
    """The exact token-causal mask (full blocks below the diagonal, one lower-
    triangular tile on it)."""
    w = W.Workload("fp8_token_causal", 1, 2, 1024, 128, 128, 128, "bf16", "token_causal")
    st, pidx, pbits = W.make_elem_mask(w)
    q, k, v = _fp8_inputs(1, 2, 1024, 128, 88)
    _run_elem(q, k, v, st, pidx, pbits, 128, 128, 1.0 / np.sqrt(128), "token-causal")


def test_fp8_elem_planned_all_full_and_empty():
    """plan_elem + fwd_fp8_planned_elem equals fwd_fp8_elem bit for bit; all-full
    states equal the block-mask fp8 forward (all ones) bit for bit; all-empty
    states give out = 0, lse = -inf."""
    ensure_built()
    B, H, S, D, b = 1, 2, 512, 128, 128
    q, k, v = (t.cuda() for t in _fp8_inputs(B, H, S, D, 23))
    st, pidx, pbits = (t.cuda() for t in _rand_elem(B, H, S, b, b, 3, 24))
    o1, l1 = bs.fwd_fp8_elem(q, k, v, st, pidx, pbits, b, b)
    ws = torch.empty(bs.fp8_workspace_size(B, H, S, D, b, b), dtype=torch.uint8, device="cuda")
    bs.plan_elem(st, pidx, pbits, S, b, b, workspace=ws)
    o2, l2 = bs.fwd_fp8_planned_elem(q, k, v, pbits, ws, b, b)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    full = torch.ones_like(st)
    o3, l3 = bs.fwd_fp8_elem(q, k, v, full, pidx, pbits, b, b)
    o4, l4 = bs.fwd_fp8(q, k, v, torch.ones(B, H, S // b, S // b, dtype=torch.uint8, device="cuda"), b, b)
    torch.cuda.synchronize()
    assert torch.equal(o3, o4) and torch.equal(l3, l4)
    o5, l5 = bs.fwd_fp8_elem(q, k, v, torch.zeros_like(st), pidx, pbits, b, b)
    torch.cuda.synchronize()
    assert torch.all(o5 == 0) and torch.all(torch.isneginf(l5))


def test_fp8_elem_workload_token_causal_sampled():
    """The exact token-causal shape (B2 H32 S8192 D128) in fp8 at full size, on
    sampled rows (the first and last rows of blocks included)."""
    w = W.ELEM_WORKLOADS["causal_elem_bf16"]
    ensure_built()
    st, pidx, pbits = W.make_elem_mask(w)
    q, k, v = _fp8_inputs(w.B, w.H, w.S, w.D, 1)
    say("fwd_fp8_elem workload", tuple(q.shape))
    out, lse = bs.fwd_fp8_elem(q.cuda(), k.cuda(), v.cuda(), st.cuda(), pidx.cuda(), pbits.cuda(),
                               w.block_q, w.block_k, w.scale)
    torch.cuda.synchronize()
    rows = W.sample_rows(w.B, w.H, w.S, w.block_q, 48)
    ro, rl = oracle.fwd_rows_elem(q, k, v, st, pidx, pbits, w.block_q, w.block_k, w.scale, rows)
    go = out.reshape(-1, w.D)[torch.as_tensor(rows, device=out.device)]
    gl = lse.reshape(-1)[torch.as_tensor(rows, device=lse.device)]
    keep = _keep_rows(st, pidx, pbits, w.block_q, w.block_k, rows, w.S)
    bound = _bound_keep(q, k, v, keep, w.scale, rows, ro)
    say("  max err", _check(go, gl, ro, rl, bound, "token-causal fp8, sampled"))


@pytest.mark.timeout(600)
def test_fp8_largest_head():
    """The largest head the boundary takes for D = 128 (S = 2^22 - 128, 32767 key
    blocks per row, 1 GiB of mask) in fp8: the diagonal, the last key block in every
    row, two random blocks per row and an empty row; sampled rows (the first and last
    among them) against their bound."""
    ensure_built()
    B, H, D, b = 1, 1, 128, 128
    S = (1 << 22) - 128
    n = S // b
    scale = 1.0 / np.sqrt(D)
    say("fwd_fp8 largest head", (B, H, S, D))
    q, k, v = _fp8_inputs(B, H, S, D, 76)
    g = torch.Generator().manual_seed(76)
    mask = torch.zeros(B, H, n, n, dtype=torch.uint8)
    i = torch.arange(n)
    mask[0, 0, i, i] = 1
    mask[0, 0, :, n - 1] = 1
    for _ in range(2):
        mask[0, 0, i, torch.randint(0, n, (n,), generator=g)] = 1
    mask[0, 0, 5] = 0
    out, lse = bs.fwd_fp8(q.cuda(), k.cuda(), v.cuda(), mask.cuda(), b, b, scale)
    torch.cuda.synchronize()
    rows = np.union1d(W.sample_rows(B, H, S, b, 24, mask=mask), [5 * b, 5 * b + 77, S - 1])
    ro, rl = oracle.fwd_rows(q, k, v, mask, b, b, scale, rows)
    # the bound of _bound_rows, row by row on the row's own keys only
    m = mask[0, 0].numpy() != 0
    bound = np.zeros((len(rows), D))
    for t, r in enumerate(rows):
        keys = torch.as_tensor(np.nonzero(np.repeat(m[r // b], b))[0])
        if keys.numel() == 0:
            continue
        kf, vf = k[0, 0][keys].double().numpy(), v[0, 0][keys].double().numpy()
        sc = float(np.float32(scale)) * (kf @ q[0, 0, r].double().numpy())
        w = np.exp(sc - sc.max())
        w /= w.sum()
        av = np.abs(vf)
        bound[t] = 2.0 ** -4 * (w @ av) + 2.0 ** -10 * w.max() * av.sum(0) + D * 2.0 ** -24 * (w @ av)
    bound = 2 * (bound + 2.0 ** -9 * np.abs(ro))
    go = out.reshape(-1, D)[torch.as_tensor(rows, device=out.device)]
    gl = lse.reshape(-1)[torch.as_tensor(rows, device=lse.device)]
    say("  max err", _check(go, gl, ro, rl, bound, "fp8 largest head"))
