"""Element-level masks on the GPU (bsattn_fwd_elem and its plan / planned steps)
against the fp64 oracle's element-mask forward on identical seeded inputs.

Block states: 0 empty, 1 full, anything else partial through a bit tile
(include/bsattn.h).  Small shapes are compared over the whole output on every
built element-mask config; the token-causal workload runs at full size on a
seeded row sample."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import bs, compare, ensure_built, rand_qkv, say

pytestmark = pytest.mark.gpu


def _rand_elem(B, H, S, bq, bk, n_tiles, seed, p=(0.3, 0.3, 0.4), density=0.5, zero_row=True):
    """Random states (empty / full / partial), random tile per block and random
    bit tiles; with zero_row, tile 0 has one all-clear row and tile 1 (if any)
    is all clear, so some query rows keep nothing in some blocks."""
    g = np.random.default_rng(seed)
    st = g.choice(3, size=(B, H, S // bq, S // bk), p=p).astype(np.uint8)
    st[st == 2] = g.choice([2, 3, 200], size=int((st == 2).sum()))
    pidx = g.integers(0, n_tiles, size=st.shape).astype(np.int32)
    bits = g.random((n_tiles, bq, bk)) < density
    if zero_row:
        bits[0, 3, :] = False
        if n_tiles > 1:
            bits[1] = False
    return torch.from_numpy(st), torch.from_numpy(pidx), W.pack_tiles(bits)


def _run(q, k, v, st, pidx, pbits, bq, bk, scale, config=None, what=""):
    ensure_built()
    say("fwd_elem", what, tuple(q.shape), q.dtype, bq, bk, config)
    out, lse = bs.fwd_elem(q.cuda(), k.cuda(), v.cuda(), st.cuda(), pidx.cuda(), pbits.cuda(),
                           bq, bk, scale, config=config)
    torch.cuda.synchronize()
    ro, rl = oracle.fwd_elem(q, k, v, st, pidx, pbits, bq, bk, scale)
    return out, lse, compare(out, lse, ro, rl, "bf16", what)


def _configs(D, bq, bk):
    ensure_built()
    return [c.as_tuple() for c in bs.list_configs_elem(torch.bfloat16, D, bq, bk)]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("blocks", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_every_config(D, blocks):
    bq, bk = blocks
    S = 512
    q, k, v = rand_qkv(1, 2, S, D, torch.bfloat16, seed=D + bq)
    st, pidx, pbits = _rand_elem(1, 2, S, bq, bk, 3, seed=bq * 7 + bk)
    cfgs = _configs(D, bq, bk)
    assert cfgs, "no element-mask config for D=%d blocks=%s" % (D, blocks)
    for cfg in cfgs:
        _run(q, k, v, st, pidx, pbits, bq, bk, 1.0 / np.sqrt(D), cfg, "%s %s" % (blocks, cfg))


@pytest.mark.parametrize("scale", ["zero", "negzero", "negative"])
@pytest.mark.parametrize("D", [64, 128])
def test_degenerate_scales_every_config(D, scale):
    """scale 0 (and -0.0) makes every kept score 0: a uniform softmax over the
    kept keys of each row (dropped scores must still give exactly nothing, not
    -inf * 0 = NaN); a negative scale (-1/sqrt(D), the workloads' magnitude)
    flips the scores.  Rows with partial blocks, a tile row that keeps nothing
    and an all-clear tile are included."""
    b, S = 128, 512
    scale = {"zero": 0.0, "negzero": -0.0, "negative": -1.0 / np.sqrt(D)}[scale]
    q, k, v = rand_qkv(1, 2, S, D, torch.bfloat16, seed=D + 17)
    st, pidx, pbits = _rand_elem(1, 2, S, b, b, 3, seed=29)
    for cfg in _configs(D, b, b):
        _run(q, k, v, st, pidx, pbits, b, b, scale, cfg, "scale %r %s" % (scale, cfg))


@pytest.mark.parametrize("D", [64, 128])
def test_token_causal(D):
    """Exact token-causal attention: full blocks below the diagonal, one shared
    lower-triangular tile on it (ragged: S = 640, five 128-blocks)."""
    B, H, S, b = 1, 3, 640, 128
    q, k, v = rand_qkv(B, H, S, D, torch.bfloat16, seed=5)
    n = S // b
    i = torch.arange(n).view(n, 1)
    j = torch.arange(n).view(1, n)
    st = ((j < i).to(torch.uint8) + 2 * (j == i).to(torch.uint8)).expand(B, H, n, n).contiguous()
    pidx = torch.zeros(B, H, n, n, dtype=torch.int32)
    pbits = W.pack_tiles(np.tril(np.ones((b, b), dtype=bool))[None])
    for cfg in _configs(D, b, b):
        _run(q, k, v, st, pidx, pbits, b, b, 1.0 / np.sqrt(D), cfg, "token causal %s" % (cfg,))


def test_all_set_tiles_equal_block_mask():
    """Partial blocks whose tiles are all ones give bit-for-bit the block-mask
    forward of the same tile config (the same arithmetic, the bit test passes)."""
    ensure_built()
    B, H, S, D, b = 1, 2, 512, 128, 128
    q, k, v = (t.cuda() for t in rand_qkv(B, H, S, D, torch.bfloat16, seed=9))
    st, pidx, _ = _rand_elem(B, H, S, b, b, 2, seed=9, zero_row=False)
    pbits = W.pack_tiles(np.ones((2, b, b), dtype=bool))
    for cfg in _configs(D, b, b):
        oe, le = bs.fwd_elem(q, k, v, st.cuda(), pidx.cuda(), pbits.cuda(), b, b, config=cfg)
        ob, lb = bs.fwd(q, k, v, (st != 0).to(torch.uint8).cuda(), b, b, config=cfg)
        torch.cuda.synchronize()
        assert torch.equal(oe, ob), cfg
        assert torch.equal(le, lb), cfg


def test_planned_matches_fwd_and_rows_without_keys():
    """plan_elem + fwd_planned_elem equals fwd_elem, and rows that keep no
    element anywhere give out = 0, lse = -inf."""
    ensure_built()
    B, H, S, D, b = 2, 1, 384, 64, 128
    q, k, v = rand_qkv(B, H, S, D, torch.bfloat16, seed=11)
    n = S // b
    st = torch.full((B, H, n, n), 2, dtype=torch.uint8)
    st[0, 0, 1, :] = 0                      # query block 1 of (0, 0): no block at all
    pidx = torch.zeros(B, H, n, n, dtype=torch.int32)
    bits = np.random.default_rng(3).random((1, b, b)) < 0.3
    bits[0, 10:20, :] = False               # queries 10..19 of every block keep nothing
    pbits = W.pack_tiles(bits)
    out, lse, _ = _run(q, k, v, st, pidx, pbits, b, b, 0.125, what="empty rows")
    l = lse.cpu()
    assert torch.all(torch.isneginf(l[0, 0, 128:256]))
    assert torch.all(torch.isneginf(l[:, :, 10:20])) and torch.all(torch.isneginf(l[:, :, 138:148]))
    assert torch.all(out.cpu()[:, :, 10:20] == 0)
    ws = bs.plan_elem(st.cuda(), pidx.cuda(), pbits.cuda(), S, b, b)
    for cfg in _configs(D, b, b):
        o1, l1 = bs.fwd_elem(q.cuda(), k.cuda(), v.cuda(), st.cuda(), pidx.cuda(), pbits.cuda(),
                             b, b, 0.125, config=cfg)
        o2, l2 = bs.fwd_planned_elem(q.cuda(), k.cuda(), v.cuda(), pbits.cuda(), ws, b, b, 0.125,
                                     config=cfg)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), cfg


def test_tile_index_out_of_range_is_clamped():
    """A partial block naming a tile past n_tiles reads the last tile (no access
    outside partial_bits); a negative index reads tile 0."""
    B, H, S, D, b = 1, 1, 256, 128, 128
    q, k, v = rand_qkv(B, H, S, D, torch.bfloat16, seed=13)
    st = torch.full((B, H, 2, 2), 2, dtype=torch.uint8)
    bits = np.random.default_rng(4).random((2, b, b)) < 0.5
    pbits = W.pack_tiles(bits)
    bad = torch.tensor([[[[5, -3], [1, 99]]]], dtype=torch.int32)
    good = torch.tensor([[[[1, 0], [1, 1]]]], dtype=torch.int32)
    ensure_built()
    o1, l1 = bs.fwd_elem(q.cuda(), k.cuda(), v.cuda(), st.cuda(), bad.cuda(), pbits.cuda(), b, b)
    o2, l2 = bs.fwd_elem(q.cuda(), k.cuda(), v.cuda(), st.cuda(), good.cuda(), pbits.cuda(), b, b)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_workload_token_causal_sampled_rows():
    """The full-size token-causal workload (B2 H32 S8192 D128) on sampled rows."""
    w = W.ELEM_WORKLOADS["causal_elem_bf16"]
    ensure_built()
    q, k, v, _ = W.make_inputs(w)
    st, pidx, pbits = W.make_elem_mask(w)
    say("workload", w.name, tuple(q.shape))
    out, lse = bs.fwd_elem(q.cuda(), k.cuda(), v.cuda(), st.cuda(), pidx.cuda(), pbits.cuda(),
                           w.block_q, w.block_k, w.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    rows = W.sample_rows(w.B, w.H, w.S, w.block_q, 48)
    ro, rl = oracle.fwd_rows_elem(q, k, v, st, pidx, pbits, w.block_q, w.block_k, w.scale, rows)
    go = out.reshape(-1, w.D)[torch.as_tensor(rows, device=out.device)]
    gl = lse.reshape(-1)[torch.as_tensor(rows, device=lse.device)]
    say("  stats", compare(go, gl, ro, rl, "bf16", w.name))


# ---- fp32 inputs -------------------------------------------------------------------

def _configs_f32(D, bq, bk):
    ensure_built()
    return [c.as_tuple() for c in bs.list_configs_elem(torch.float32, D, bq, bk)]


def _run_f32(q, k, v, st, pidx, pbits, bq, bk, scale, config=None, what=""):
    ensure_built()
    say("fwd_elem fp32", what, tuple(q.shape), bq, bk, config)
    out, lse = bs.fwd_elem(q.cuda(), k.cuda(), v.cuda(), st.cuda(), pidx.cuda(), pbits.cuda(),
                           bq, bk, scale, config=config)
    torch.cuda.synchronize()
    assert out.dtype == torch.float32
    ro, rl = oracle.fwd_elem(q, k, v, st, pidx, pbits, bq, bk, scale)
    return out, lse, compare(out, lse, ro, rl, "f32", what)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("blocks", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_fp32_every_config(D, blocks):
    """fp32 inputs (the fp32 kernel, fp32 tolerances) on every built config."""
    bq, bk = blocks
    S = 512
    q, k, v = rand_qkv(1, 2, S, D, torch.float32, seed=D + bq + 1)
    st, pidx, pbits = _rand_elem(1, 2, S, bq, bk, 3, seed=bq * 7 + bk + 1)
    cfgs = _configs_f32(D, bq, bk)
    assert cfgs, "no fp32 element-mask config for D=%d blocks=%s" % (D, blocks)
    for cfg in cfgs:
        _run_f32(q, k, v, st, pidx, pbits, bq, bk, 1.0 / np.sqrt(D), cfg, "%s %s" % (blocks, cfg))


@pytest.mark.parametrize("scale", [0.0, -0.3])
def test_fp32_token_causal_and_degenerate_scales(scale):
    """fp32 exact token-causal (ragged: S = 640) with the default scale, then a zero
    scale (uniform over the kept keys) and a negative one on random tiles."""
    B, H, S, b, D = 1, 2, 640, 128, 64
    q, k, v = rand_qkv(B, H, S, D, torch.float32, seed=15)
    n = S // b
    i = torch.arange(n).view(n, 1)
    j = torch.arange(n).view(1, n)
    st = ((j < i).to(torch.uint8) + 2 * (j == i).to(torch.uint8)).expand(B, H, n, n).contiguous()
    pidx = torch.zeros(B, H, n, n, dtype=torch.int32)
    pbits = W.pack_tiles(np.tril(np.ones((b, b), dtype=bool))[None])
    _run_f32(q, k, v, st, pidx, pbits, b, b, 1.0 / np.sqrt(D), what="fp32 token causal")
    st2, pidx2, pbits2 = _rand_elem(B, H, S, 128, 64, 3, seed=16)
    _run_f32(q, k, v, st2, pidx2, pbits2, 128, 64, scale, what="fp32 scale %g" % scale)


def test_fp32_all_set_tiles_equal_block_mask():
    """fp32: all-set tiles give bit for bit the block-mask forward of the same config."""
    ensure_built()
    B, H, S, D, b = 1, 2, 512, 128, 128
    q, k, v = (t.cuda() for t in rand_qkv(B, H, S, D, torch.float32, seed=19))
    st, pidx, _ = _rand_elem(B, H, S, b, b, 2, seed=19, zero_row=False)
    pbits = W.pack_tiles(np.ones((2, b, b), dtype=bool))
    for cfg in _configs_f32(D, b, b):
        oe, le = bs.fwd_elem(q, k, v, st.cuda(), pidx.cuda(), pbits.cuda(), b, b, config=cfg)
        ob, lb = bs.fwd(q, k, v, (st != 0).to(torch.uint8).cuda(), b, b, config=cfg)
        torch.cuda.synchronize()
        assert torch.equal(oe, ob), cfg
        assert torch.equal(le, lb), cfg
