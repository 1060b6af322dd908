"""Backward on the GPU (bsattn_bwd and its plan / planned steps) against the fp64
oracle's backward on identical seeded bf16 inputs.

The GPU gradients start from the GPU forward's out and lse (as a training step
would); the oracle recomputes everything from q, k, v and dout in fp64.

Tolerance, per element, derived from the arithmetic (u = 2^-9, the relative
rounding bound of bf16):
  - P is rounded to bf16 before dV += dO^T P: |err dv_j| <= u sum_r P_rj |dout_r|;
  - delta is dout . out with the forward's bf16 out, whose own error is at most
    2u sum_j P_rj |v_j| (its P in bf16) + u |out_r| (its rounding):
    E_r = sum_d |dout_rd| (2u (P|v|)_rd + u |out_rd|);
  - dS = P (dP - delta) is rounded to bf16 before dK += Q^T dS and dQ += dS K, and
    dP is an fp32 sum of D exact products: |err dS_rj| <= u |dS_rj| + P_rj (E_r +
    D 2^-24 (|dout| |v|^T)_rj);
  - |err dk_j| <= |scale| sum_r |err dS_rj| |q_r|, |err dq_r| <= |scale| sum_j
    |err dS_rj| |k_j|;
  - fp32 accumulation adds n 2^-24 of the absolute sum (n terms), and a bf16
    gradient adds u |g|.
Every element is held to twice that bound (the exp2 and the fp32 sums add a few
ulp more), and the mean error must stay well below the mean bound."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import bs, ensure_built, rand_mask, rand_qkv, say

pytestmark = pytest.mark.gpu

U = 2.0 ** -9


def _bounds(q, k, v, do, out, full, scale, grad_bf16):
    """Per-element error bounds [B,H,S,D] for dq, dk, dv (fp64 numpy) from the
    magnitudes of the exact quantities; full is the [B,H,S,S] element mask."""
    q, k, v, do, out = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do, out))
    D = q.shape[-1]
    s = float(np.float32(scale)) * (q @ np.swapaxes(k, -1, -2))
    s = np.where(full, s, -np.inf)
    anyk = full.any(-1, keepdims=True)
    m = np.where(anyk, s.max(-1, keepdims=True), 0.0)
    e = np.where(full, np.exp(s - m), 0.0)
    l = e.sum(-1, keepdims=True)
    P = np.where(anyk, e / np.where(l > 0, l, 1.0), 0.0)
    dP = do @ np.swapaxes(v, -1, -2)
    delta = (P * dP).sum(-1, keepdims=True)
    dS = P * (dP - delta)
    av, ado, aq, ak = np.abs(v), np.abs(do), np.abs(q), np.abs(k)
    E = (ado * (2 * U * (P @ av) + U * np.abs(out))).sum(-1, keepdims=True)
    dp_err = D * 2.0 ** -24 * (ado @ np.swapaxes(av, -1, -2))
    ds_err = U * np.abs(dS) + P * (E + dp_err) + 2.0 ** -20 * np.abs(dS)
    n = full.shape[-1]
    acc = n * 2.0 ** -24
    sc = abs(float(np.float32(scale)))
    PT = np.swapaxes(P, -1, -2)
    b_dv = U * (PT @ ado) + acc * (PT @ ado)
    b_dk = sc * (np.swapaxes(ds_err, -1, -2) @ aq) + acc * sc * (np.swapaxes(np.abs(dS), -1, -2) @ aq)
    b_dq = sc * (ds_err @ ak) + acc * sc * (np.abs(dS) @ ak)
    return 2 * b_dq, 2 * b_dk, 2 * b_dv


def _check(name, got, ref, bound, grad_bf16, what):
    got = got.double().cpu().numpy()
    b = bound + (2 * U * np.abs(ref) if grad_bf16 else 0.0) + 1e-30
    err = np.abs(got - ref)
    assert not np.isnan(got).any(), (what, name, "NaN")
    bad = err > b
    assert not bad.any(), (what, name, int(bad.sum()), float((err - b).max()), float(err[bad].max()))
    assert err.mean() <= 0.5 * b.mean(), (what, name, float(err.mean()), float(b.mean()))
    return float(err.max())


def _run(B, H, S, D, bq, bk, scale, seed, grad_dtype, p=0.5, what="", global_cols=()):
    ensure_built()
    q, k, v = rand_qkv(B, H, S, D, torch.bfloat16, seed)
    g = torch.Generator().manual_seed(seed + 1)
    do = torch.randn(B, H, S, D, generator=g).to(torch.bfloat16)
    mask = rand_mask(B, H, S // bq, S // bk, p, seed, diag=False, empty_rows=[(0, 0, 1)])
    for c in global_cols:  # key blocks every query block sees (but the empty row)
        mask[:, :, :, c] = 1
        mask[0, 0, 1, :] = 0
    mask[0, -1, :, 0] = 0  # key block 0 of the last head: seen by no query block
    say("bwd", what, (B, H, S, D), (bq, bk), scale, grad_dtype)
    qd, kd, vd, dod, md = (t.cuda() for t in (q, k, v, do, mask))
    out, lse = bs.fwd(qd, kd, vd, md, bq, bk, scale)
    gq, gk, gv = bs.bwd(qd, kd, vd, out, lse, dod, md, bq, bk, scale, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.bwd(q, k, v, do, mask, bq, bk, scale)
    full = np.repeat(np.repeat(mask.numpy() != 0, bq, axis=2), bk, axis=3)
    bf = grad_dtype == torch.bfloat16
    bq_, bk_, bv_ = _bounds(q.float(), k.float(), v.float(), do.float(), out.float().cpu(), full, scale, bf)
    stats = {n: _check(n, g_, r, b, bf, what) for n, g_, r, b in
             (("dq", gq, rq, bq_), ("dk", gk, rk, bk_), ("dv", gv, rv, bv_))}
    # rows that see no key and keys no row sees: exact zeros
    assert torch.all(gq[0, 0, bq:2 * bq] == 0)
    assert torch.all(gk[0, -1, :bk] == 0) and torch.all(gv[0, -1, :bk] == 0)
    say("  max err", stats)
    return gq, gk, gv


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("blocks", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_bwd_small(D, blocks):
    bq, bk = blocks
    _run(1, 2, 512, D, bq, bk, 1.0 / np.sqrt(D), 7 + D + bq, torch.bfloat16, what="%s" % (blocks,))


@pytest.mark.parametrize("D", [64, 128])
def test_bwd_fp32_grads_negative_scale(D):
    _run(2, 1, 384, D, 128, 64, -0.3, 21 + D, torch.float32, p=0.6, what="fp32 grads")


def test_bwd_dense_and_empty_mask():
    """All blocks active (every key seen by every row), and an all-zero mask
    (every gradient exactly 0)."""
    _run(1, 2, 256, 128, 128, 128, 0.09, 31, torch.bfloat16, p=1.1, what="dense")
    ensure_built()
    B, H, S, D = 1, 1, 256, 64
    q, k, v = (t.cuda() for t in rand_qkv(B, H, S, D, torch.bfloat16, 3))
    mask = torch.zeros(B, H, 2, 2, dtype=torch.uint8, device="cuda")
    out, lse = bs.fwd(q, k, v, mask, 128, 128)
    g = bs.bwd(q, k, v, out, lse, q, mask, 128, 128)
    torch.cuda.synchronize()
    for t in g:
        assert torch.all(t == 0)


def test_bwd_planned_deterministic():
    """bwd_plan + bwd_planned equals bwd bit for bit, and repeated calls agree bit
    for bit (no atomics, fixed summation order)."""
    ensure_built()
    B, H, S, D, b = 2, 2, 512, 128, 128
    q, k, v = (t.cuda() for t in rand_qkv(B, H, S, D, torch.bfloat16, 41))
    do = torch.randn(B, H, S, D, device="cuda").to(torch.bfloat16)
    mask = rand_mask(B, H, S // b, S // b, 0.6, 41).cuda()
    out, lse = bs.fwd(q, k, v, mask, b, b)
    g1 = bs.bwd(q, k, v, out, lse, do, mask, b, b)
    ws = bs.bwd_plan(mask, S, b, b)
    g2 = bs.bwd_planned(q, k, v, out, lse, do, ws, b, b)
    g3 = bs.bwd_planned(q, k, v, out, lse, do, ws, b, b)
    torch.cuda.synchronize()
    for a, c, d in zip(g1, g2, g3):
        assert torch.equal(a, c) and torch.equal(c, d)


def test_bwd_workload_dense_sampled():
    """The dense workload (B4 H16 S2048 D128, 128x128 blocks) at full size: every
    row of two heads held to the bound, the oracle on a sample of rows."""
    w = W.WORKLOADS["dense_bf16"]
    ensure_built()
    q, k, v, mask = W.make_inputs(w)
    g = torch.Generator().manual_seed(99)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    dev = [t.cuda() for t in (q, k, v, do, mask)]
    say("bwd workload", w.name, tuple(q.shape))
    out, lse = bs.fwd(dev[0], dev[1], dev[2], dev[4], w.block_q, w.block_k, w.scale)
    gq, gk, gv = bs.bwd(dev[0], dev[1], dev[2], out, lse, dev[3], dev[4], w.block_q, w.block_k, w.scale)
    torch.cuda.synchronize()
    for t in (gq, gk, gv):
        assert torch.isfinite(t.float()).all()
    S, D = w.S, w.D
    rng = np.random.default_rng(5)
    for bh in (0, w.B * w.H - 1):
        rows = bh * S + np.sort(rng.choice(S, 24, replace=False))
        rq, rk, rv = oracle.bwd_sample(q, k, v, do, mask, w.block_q, w.block_k, w.scale, rows, rows)
        b_, h_ = divmod(bh, w.H)
        full = np.repeat(np.repeat(mask[b_, h_].numpy() != 0, w.block_q, 0), w.block_k, 1)
        bnd = _bounds(q[b_, h_].float(), k[b_, h_].float(), v[b_, h_].float(), do[b_, h_].float(),
                      out[b_, h_].float().cpu(), full, w.scale, True)
        loc = rows - bh * S
        for name, gg, r, bb in (("dq", gq, rq, bnd[0]), ("dk", gk, rk, bnd[1]), ("dv", gv, rv, bnd[2])):
            got = gg.reshape(-1, D)[torch.as_tensor(rows, device="cuda")]
            _check(name, got, r, bb[loc], True, "%s head %d" % (w.name, bh))


@pytest.mark.timeout(600)
def test_bwd_workload_dense_full():
    """The dense workload (B4 H16 S2048 D128, 128x128 blocks) at full size: every
    element of dq, dk and dv against the oracle's full backward, each held to its
    bound (computed one head at a time)."""
    import time
    w = W.WORKLOADS["dense_bf16"]
    ensure_built()
    q, k, v, mask = W.make_inputs(w)
    g = torch.Generator().manual_seed(99)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    dev = [t.cuda() for t in (q, k, v, do, mask)]
    say("bwd workload, full output", w.name, tuple(q.shape))
    out, lse = bs.fwd(dev[0], dev[1], dev[2], dev[4], w.block_q, w.block_k, w.scale)
    gq, gk, gv = bs.bwd(dev[0], dev[1], dev[2], out, lse, dev[3], dev[4], w.block_q, w.block_k, w.scale)
    torch.cuda.synchronize()
    gq, gk, gv, out = gq.cpu(), gk.cpu(), gv.cpu(), out.cpu()
    say("oracle bwd, full output on", oracle.max_threads(), "threads ...")
    t0 = time.perf_counter()
    rq, rk, rv = oracle.bwd(q, k, v, do, mask, w.block_q, w.block_k, w.scale)
    say("oracle bwd done in %.1f s" % (time.perf_counter() - t0))
    full = np.ones((w.S, w.S), dtype=bool)  # every block active
    assert bool(mask.all())
    worst = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for bh in range(w.B * w.H):
        b_, h_ = divmod(bh, w.H)
        bnd = _bounds(q[b_, h_].float(), k[b_, h_].float(), v[b_, h_].float(), do[b_, h_].float(),
                      out[b_, h_].float(), full, w.scale, True)
        for name, gg, r, bb in (("dq", gq, rq, bnd[0]), ("dk", gk, rk, bnd[1]), ("dv", gv, rv, bnd[2])):
            e = _check(name, gg[b_, h_], r[b_, h_], bb, True, "%s head %d" % (w.name, bh))
            worst[name] = max(worst[name], e)
    say("  max err over all elements", worst)


def test_bwd_parts():
    """parts = PREP | DKDV writes dk, dv only (dq untouched) and equals the full
    call; DQ alone on that workspace then gives the full call's dq."""
    ensure_built()
    B, H, S, D, bq, bk = 1, 2, 512, 64, 64, 128
    q, k, v = (t.cuda() for t in rand_qkv(B, H, S, D, torch.bfloat16, 51))
    do = torch.randn(B, H, S, D, device="cuda").to(torch.bfloat16)
    mask = rand_mask(B, H, S // bq, S // bk, 0.5, 51).cuda()
    out, lse = bs.fwd(q, k, v, mask, bq, bk)
    full = bs.bwd(q, k, v, out, lse, do, mask, bq, bk)
    ws = bs.bwd_plan(mask, S, bq, bk)
    sentinel = torch.full_like(q, 7.0)
    dq = sentinel.clone()
    _, dk, dv = bs.bwd_planned(q, k, v, out, lse, do, ws, bq, bk, dq=dq, parts=bs.BWD_PREP | bs.BWD_DKDV)
    torch.cuda.synchronize()
    assert torch.equal(dq, sentinel)
    assert torch.equal(dk, full[1]) and torch.equal(dv, full[2])
    dk2, dv2 = sentinel.clone(), sentinel.clone()
    dq2, _, _ = bs.bwd_planned(q, k, v, out, lse, do, ws, bq, bk, dk=dk2, dv=dv2, parts=bs.BWD_DQ)
    torch.cuda.synchronize()
    assert torch.equal(dq2, full[0])
    assert torch.equal(dk2, sentinel) and torch.equal(dv2, sentinel)


@pytest.mark.parametrize("D", [64, 128])
def test_bwd_cut_key_blocks(D):
    """Key blocks seen by every query block are cut into pieces (partial sums in
    fp32 scratch, added in piece order): S 2048 with 64-blocks gives 32 query
    blocks per column, far above the piece length, on two global columns."""
    _run(1, 2, 2048, D, 64, 64, 1.0 / np.sqrt(D), 61 + D, torch.bfloat16, p=0.15, what="cut columns",
         global_cols=(1, 2))
    ensure_built()
    B, H, S, b = 1, 2, 2048, 64
    q, k, v = (t.cuda() for t in rand_qkv(B, H, S, D, torch.bfloat16, 62))
    do = torch.randn(B, H, S, D, device="cuda").to(torch.bfloat16)
    mask = rand_mask(B, H, S // b, S // b, 0.15, 62).cuda()
    mask[:, :, :, 3] = 1
    out, lse = bs.fwd(q, k, v, mask, b, b)
    g1 = bs.bwd(q, k, v, out, lse, do, mask, b, b)
    g2 = bs.bwd(q, k, v, out, lse, do, mask, b, b)
    torch.cuda.synchronize()
    for x, y in zip(g1, g2):
        assert torch.equal(x, y)


def _key_bounds(dev, out, lse, mask, b, scale, j):
    """The bounds of _bounds for dk_j and dv_j of one key of head 0 (fp64 torch on the
    device, rows in chunks): every query row that sees the key contributes; P from
    the forward's lse; the row's sum over keys of P |v| is bounded by max |v| (sum P
    = 1), so the bound is looser than _bounds', never tighter."""
    q, k, v, do = (t[0, 0] for t in dev[:4])
    D = q.shape[-1]
    blocks = torch.nonzero(mask[:, j // b]).flatten()
    rows = (blocks[:, None] * b + torch.arange(b, device=q.device)).flatten()
    sc = float(np.float32(scale))
    vmax = v.double().abs().max(0).values
    kj, vj = k[j].double(), v[j].double()
    sum_dk_err = torch.zeros(D, dtype=torch.float64, device=q.device)
    sum_ds_q = torch.zeros_like(sum_dk_err)
    sum_p_do = torch.zeros_like(sum_dk_err)
    for c in range(0, rows.numel(), 1 << 20):
        r = rows[c:c + (1 << 20)]
        qr, dor, outr = q[r].double(), do[r].double(), out[0, 0][r].double()
        P = torch.exp(sc * (qr @ kj) - lse[0, 0][r].double())
        dS = P * (dor @ vj - (dor * outr).sum(1))
        E = (dor.abs() * (2 * U * vmax + U * outr.abs())).sum(1)
        dp_err = D * 2.0 ** -24 * (dor.abs() @ vj.abs())
        ds_err = U * dS.abs() + P * (E + dp_err) + 2.0 ** -20 * dS.abs()
        sum_dk_err += (ds_err[:, None] * qr.abs()).sum(0)
        sum_ds_q += (dS.abs()[:, None] * qr.abs()).sum(0)
        sum_p_do += (P[:, None] * dor.abs()).sum(0)
    acc = rows.numel() * 2.0 ** -24
    b_dk = 2 * abs(sc) * (sum_dk_err + acc * sum_ds_q)
    b_dv = 2 * (U + acc) * sum_p_do
    return b_dk.cpu().numpy(), b_dv.cpu().numpy()


@pytest.mark.timeout(900)
def test_bwd_largest_head():
    """The backward at the largest head the boundary takes for D = 128 (S = 2^22 -
    128: 32767 key blocks per row, 1 GiB of mask): the diagonal, two random blocks
    per row, an empty row, and the last key block seen by every query block, so its
    column is cut into 256 pieces whose partial sums the reduce kernel adds.  dq on
    sampled rows (the first and last among them), dk and dv on sampled keys (the
    last key among them), each held to its bound against the oracle."""
    ensure_built()
    B, H, D, b = 1, 1, 128, 128
    S = (1 << 22) - 128
    n = S // b
    scale = 1.0 / np.sqrt(D)
    say("bwd largest head", (B, H, S, D))
    q, k, v = rand_qkv(B, H, S, D, torch.bfloat16, seed=74)
    do = torch.randn(B, H, S, D, generator=torch.Generator().manual_seed(75)).to(torch.bfloat16)
    g = torch.Generator().manual_seed(74)
    mask = torch.zeros(B, H, n, n, dtype=torch.uint8)
    i = torch.arange(n)
    mask[0, 0, i, i] = 1
    mask[0, 0, :, n - 1] = 1
    for _ in range(2):
        mask[0, 0, i, torch.randint(0, n, (n,), generator=g)] = 1
    mask[0, 0, 5] = 0
    dev = [t.cuda() for t in (q, k, v, do, mask)]
    out, lse = bs.fwd(dev[0], dev[1], dev[2], dev[4], b, b, scale)
    gq, gk, gv = bs.bwd(dev[0], dev[1], dev[2], out, lse, dev[3], dev[4], b, b, scale)
    torch.cuda.synchronize()
    assert torch.all(gq[0, 0, 5 * b:6 * b] == 0)
    rng = np.random.default_rng(74)
    q_rows = np.union1d(rng.choice(S, 14, replace=False), [0, 5 * b + 3, S - 1])
    k_rows = np.union1d(rng.choice(S - b, 5, replace=False), [0, S - b, S - 1])
    say("  oracle on", len(q_rows), "rows and", len(k_rows), "keys,", oracle.max_threads(), "threads")
    rq, rk, rv = oracle.bwd_sample(q, k, v, do, mask, b, b, scale, q_rows, k_rows)
    m = mask[0, 0].numpy() != 0
    out_c = out[0, 0].float().cpu()
    # dq bound: the sampled rows with every key (row-local quantities only)
    fq = np.repeat(m[q_rows // b], b, axis=1)
    bq_ = _bounds(q[0, 0].float()[q_rows], k[0, 0].float(), v[0, 0].float(), do[0, 0].float()[q_rows],
                  out_c[q_rows], fq, scale, True)[0]
    _check("dq", gq[0, 0][torch.as_tensor(q_rows, device="cuda")], rq, bq_, True, "largest head")
    # dk, dv: the bound of _bounds per key, over every query row that sees it
    for t, j in enumerate(k_rows):
        b_k, b_v = _key_bounds(dev, out, lse, dev[4][0, 0], b, scale, int(j))
        _check("dk", gk[0, 0, j:j + 1], rk[t:t + 1], b_k[None], True, "largest head key %d" % j)
        _check("dv", gv[0, 0, j:j + 1], rv[t:t + 1], b_v[None], True, "largest head key %d" % j)
    say("  done")
