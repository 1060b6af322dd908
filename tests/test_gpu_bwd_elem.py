"""Backward with element-level masks on the GPU (bsattn_bwd_elem) against the fp64
oracle's element-mask backward on identical seeded bf16 inputs, from the GPU
element-mask forward's out and lse.  The per-element bounds are those of the
block-mask backward (tests/test_gpu_bwd.py) evaluated on the element mask: a
dropped pair contributes an exact zero on both sides."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from brute import expand_elem
from gpu_util import bs, ensure_built, rand_qkv, say
from test_gpu_bwd import _bounds, _check
from test_gpu_elem import _rand_elem

pytestmark = pytest.mark.gpu


def _run(B, H, S, D, bq, bk, scale, st, pidx, pbits, seed, grad_dtype=torch.bfloat16, what=""):
    ensure_built()
    q, k, v = rand_qkv(B, H, S, D, torch.bfloat16, seed)
    g = torch.Generator().manual_seed(seed + 1)
    do = torch.randn(B, H, S, D, generator=g).to(torch.bfloat16)
    say("bwd_elem", what, (B, H, S, D), (bq, bk), scale, grad_dtype)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    sd, pd, bd = st.cuda(), pidx.cuda(), pbits.cuda()
    out, lse = bs.fwd_elem(qd, kd, vd, sd, pd, bd, bq, bk, scale)
    gq, gk, gv = bs.bwd_elem(qd, kd, vd, out, lse, dod, sd, pd, bd, bq, bk, scale, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.bwd_elem(q, k, v, do, st, pidx, pbits, bq, bk, scale)
    full = expand_elem(st.numpy(), pidx.numpy(), pbits.numpy().view(np.uint32), bq, bk)
    bf = grad_dtype == torch.bfloat16
    b_q, b_k, b_v = _bounds(q.float(), k.float(), v.float(), do.float(), out.float().cpu(), full, scale, bf)
    stats = {n: _check(n, g_, r, b, bf, what) for n, g_, r, b in
             (("dq", gq, rq, b_q), ("dk", gk, rk, b_k), ("dv", gv, rv, b_v))}
    # rows that keep nothing and keys that no row keeps: exact zeros
    keeps_row = torch.from_numpy(full.any(-1))
    keeps_key = torch.from_numpy(full.any(-2))
    assert torch.all(gq.cpu()[~keeps_row] == 0)
    assert torch.all(gk.cpu()[~keeps_key] == 0) and torch.all(gv.cpu()[~keeps_key] == 0)
    say("  max err", stats, "rows keeping nothing", int((~keeps_row).sum()))
    return full


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("blocks", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_bwd_elem_random(D, blocks):
    bq, bk = blocks
    S = 512
    st, pidx, pbits = _rand_elem(1, 2, S, bq, bk, 3, seed=5 * bq + bk + D)
    # query block 0 of head 0 sees one partial block through tile 0, whose row 3 is
    # clear: that query keeps nothing
    st[0, 0, 0, :] = 0
    st[0, 0, 0, 0] = 2
    pidx[0, 0, 0, 0] = 0
    full = _run(1, 2, S, D, bq, bk, 1.0 / np.sqrt(D), st, pidx, pbits, seed=D + bq + 3 * bk, what="%s" % (blocks,))
    assert not full.any(-1).all()  # the case includes rows that keep nothing


def _token_causal(B, H, S, b):
    n = S // b
    st = torch.from_numpy(np.broadcast_to(np.tril(np.ones((n, n), dtype=np.uint8)) + np.eye(n, dtype=np.uint8),
                                          (B, H, n, n)).copy())
    pidx = torch.zeros((B, H, n, n), dtype=torch.int32)
    return st, pidx, W.pack_tiles(np.tril(np.ones((1, b, b), dtype=bool)))


@pytest.mark.parametrize("D", [64, 128])
def test_bwd_elem_token_causal(D):
    """Exact token-causal: full blocks below the diagonal, one shared
    lower-triangular tile on it."""
    st, pidx, pbits = _token_causal(2, 2, 512, 128)
    _run(2, 2, 512, D, 128, 128, 1.0 / np.sqrt(D), st, pidx, pbits, seed=40 + D, what="token causal")


def test_bwd_elem_fp32_grads_negative_scale():
    st, pidx, pbits = _rand_elem(2, 1, 384, 128, 64, 4, seed=77, p=(0.2, 0.3, 0.5))
    _run(2, 1, 384, 128, 128, 64, -0.3, st, pidx, pbits, seed=78, grad_dtype=torch.float32, what="fp32 grads")


def test_bwd_elem_all_full_equals_block_backward():
    """States 0/1 only (no partial block): bit for bit the block-mask backward."""
    ensure_built()
    B, H, S, D, b = 1, 2, 256, 128, 64
    q, k, v = (t.cuda() for t in rand_qkv(B, H, S, D, torch.bfloat16, 91))
    do = torch.randn(B, H, S, D, generator=torch.Generator().manual_seed(92)).to(torch.bfloat16).cuda()
    g = np.random.default_rng(93)
    st = torch.from_numpy((g.random((B, H, S // b, S // b)) < 0.6).astype(np.uint8)).cuda()
    pidx = torch.zeros(st.shape, dtype=torch.int32, device="cuda")
    pbits = torch.zeros((1, b, b // 32), dtype=torch.int32, device="cuda")
    out, lse = bs.fwd(q, k, v, st, b, b, 0.125)
    a = bs.bwd(q, k, v, out, lse, do, st, b, b, 0.125)
    e = bs.bwd_elem(q, k, v, out, lse, do, st, pidx, pbits, b, b, 0.125)
    torch.cuda.synchronize()
    for x, y in zip(a, e):
        assert torch.equal(x, y)


def test_bwd_planned_elem_equals_one_shot():
    """bsattn_bwd_plan (on the block states) + bsattn_bwd_planned_elem gives bit for
    bit the result of bsattn_bwd_elem."""
    ensure_built()
    B, H, S, D, bq, bk = 1, 2, 384, 64, 128, 64
    st, pidx, pbits = _rand_elem(B, H, S, bq, bk, 3, seed=61)
    q, k, v = (t.cuda() for t in rand_qkv(B, H, S, D, torch.bfloat16, 62))
    do = torch.randn(B, H, S, D, generator=torch.Generator().manual_seed(63)).to(torch.bfloat16).cuda()
    sd, pd, bd = st.cuda(), pidx.cuda(), pbits.cuda()
    out, lse = bs.fwd_elem(q, k, v, sd, pd, bd, bq, bk, 0.2)
    a = bs.bwd_elem(q, k, v, out, lse, do, sd, pd, bd, bq, bk, 0.2)
    ws = bs.bwd_plan(sd, S, bq, bk)
    b = bs.bwd_planned_elem(q, k, v, out, lse, do, sd, pd, bd, ws, bq, bk, 0.2)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_elem_workload_sampled():
    """The exact token-causal workload (B2 H32 S8192 D128) at full size, in the
    launch configuration bench.py times: sampled rows of the last head against the
    oracle, each held to its bound."""
    w = W.ELEM_WORKLOADS["causal_elem_bf16"]
    ensure_built()
    q, k, v, _ = W.make_inputs(w)
    st, pidx, pbits = W.make_elem_mask(w)
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(99)).to(torch.bfloat16)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    sd, pd, bd = st.cuda(), pidx.cuda(), pbits.cuda()
    say("bwd_elem workload", w.name, tuple(q.shape))
    out, lse = bs.fwd_elem(qd, kd, vd, sd, pd, bd, w.block_q, w.block_k, w.scale)
    gq, gk, gv = bs.bwd_elem(qd, kd, vd, out, lse, dod, sd, pd, bd, w.block_q, w.block_k, w.scale)
    torch.cuda.synchronize()
    for t in (gq, gk, gv):
        assert torch.isfinite(t.float()).all()
    S, D = w.S, w.D
    bh = w.B * w.H - 1
    b_, h_ = divmod(bh, w.H)
    rng = np.random.default_rng(7)
    loc = np.sort(np.concatenate([[0, 1, 127, 128, S - 1], rng.choice(S, 19, replace=False)]))
    loc = np.unique(loc)
    rows = bh * S + loc
    rq, rk, rv = oracle.bwd_sample_elem(q, k, v, do, st, pidx, pbits, w.block_q, w.block_k, w.scale, rows, rows)
    full = np.tril(np.ones((S, S), dtype=bool))  # the workload's element mask: key <= query
    bnd = _bounds(q[b_, h_].float(), k[b_, h_].float(), v[b_, h_].float(), do[b_, h_].float(),
                  out[b_, h_].float().cpu(), full, w.scale, True)
    for name, gg, r, bb in (("dq", gq, rq, bnd[0]), ("dk", gk, rk, bnd[1]), ("dv", gv, rv, bnd[2])):
        got = gg.reshape(-1, D)[torch.as_tensor(rows, device="cuda")]
        _check(name, got, r, bb[loc], True, "%s head %d" % (w.name, bh))
