"""GPU forward vs the fp64 CPU oracle on identical seeded inputs.

Small shapes are compared element by element over the whole output; the five
workloads run at full size in the default launch configuration and are compared
on a seeded sample of rows the oracle computes one by one (plus properties that
hold for every row)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import bs, compare, dkey, ensure_built, rand_mask, rand_qkv, say

pytestmark = pytest.mark.gpu


def _run_full(q, k, v, mask, bq, bk, scale, config=None, what=""):
    ensure_built()
    say("fwd", what, tuple(q.shape), q.dtype, bq, bk, scale, config)
    out, lse = bs.fwd(q.cuda(), k.cuda(), v.cuda(), mask.cuda(), bq, bk, scale, config=config)
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(q, k, v, mask, bq, bk, scale)
    return compare(out, lse, ro, rl, dkey(q), what)


@pytest.mark.parametrize("name", W.ORDER)
def test_workload_sampled_rows(name):
    w = W.WORKLOADS[name]
    ensure_built()
    q, k, v, mask = W.make_inputs(w)
    say("workload", name, tuple(q.shape), int(mask.sum()))
    out, lse = bs.fwd(q.cuda(), k.cuda(), v.cuda(), mask.cuda(), w.block_q, w.block_k, w.scale)
    torch.cuda.synchronize()
    # properties of every row: finite, no NaN, |out| bounded by max |v|
    o = out.float()
    assert torch.isfinite(o).all()
    assert torch.isfinite(lse).all()  # no workload has an empty mask row
    assert float(o.abs().max()) <= float(v.float().abs().max()) + 1e-2
    rows = W.sample_rows(w.B, w.H, w.S, w.block_q, 64, mask=mask)
    ro, rl = oracle.fwd_rows(q, k, v, mask, w.block_q, w.block_k, w.scale, rows)
    go = out.reshape(-1, w.D)[torch.as_tensor(rows, device=out.device)]
    gl = lse.reshape(-1)[torch.as_tensor(rows, device=lse.device)]
    stats = compare(go, gl, ro, rl, w.dtype, name)
    say("  stats", stats)
    if name == "tiny_f32":  # small enough for the whole output
        _run_full(q, k, v, mask, w.block_q, w.block_k, w.scale, what=name)


SHAPES = [
    # B, H, S, D, bq, bk, dtype, p
    (1, 2, 256, 64, 64, 64, torch.float32, 0.5),
    (1, 2, 384, 128, 128, 128, torch.bfloat16, 0.6),
    (2, 1, 320, 64, 64, 64, torch.bfloat16, 0.5),     # n_q = n_k = 5
    (1, 3, 512, 128, 64, 128, torch.bfloat16, 0.5),   # block_q != block_k
    (1, 2, 512, 64, 128, 64, torch.bfloat16, 0.5),
    (1, 1, 1024, 128, 128, 128, torch.bfloat16, 1.0),  # dense, 8 key blocks per row
    (2, 2, 256, 128, 64, 64, torch.float32, 0.4),
    (1, 2, 384, 64, 128, 64, torch.float32, 0.5),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(str(x) for x in s[:6]) + str(s[6])[-4:])
def test_full_output_default_config(shape):
    B, H, S, D, bq, bk, dt, p = shape
    q, k, v = rand_qkv(B, H, S, D, dt, seed=S + D)
    mask = rand_mask(B, H, S // bq, S // bk, p, seed=7, diag=True, empty_rows=[(0, 0, 1)])
    _run_full(q, k, v, mask, bq, bk, 1.0 / np.sqrt(D), what=str(shape))


def _configs(dtype, D, bq, bk):
    ensure_built()
    return [c.as_tuple() for c in bs.list_configs(dtype, D, bq, bk)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("blocks", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_every_config(dtype, D, blocks):
    bq, bk = blocks
    B, H, S = 1, 2, 512
    q, k, v = rand_qkv(B, H, S, D, dtype, seed=D + bq)
    mask = rand_mask(B, H, S // bq, S // bk, 0.5, seed=bk, empty_rows=[(0, 1, 0)])
    ro, rl = oracle.fwd(q, k, v, mask, bq, bk, 0.1)
    qd, kd, vd, md = q.cuda(), k.cuda(), v.cuda(), mask.cuda()
    cfgs = _configs(dtype, D, bq, bk)
    assert cfgs
    for cfg in cfgs:
        say("config", cfg, D, blocks, dtype)
        out, lse = bs.fwd(qd, kd, vd, md, bq, bk, 0.1, config=cfg)
        torch.cuda.synchronize()
        compare(out, lse, ro, rl, dkey(q), str(cfg))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_edge_cases(dtype):
    B, H, S, D, b = 2, 2, 256, 64, 64
    q, k, v = rand_qkv(B, H, S, D, dtype, seed=3)
    n = S // b
    # all-empty mask: zeros and -inf everywhere
    _run_full(q, k, v, torch.zeros(B, H, n, n, dtype=torch.uint8), b, b, 0.125, what="empty")
    # one active block per row, a different block per head
    m = torch.zeros(B, H, n, n, dtype=torch.uint8)
    for h in range(H):
        for i in range(n):
            m[:, h, i, (i + h) % n] = 1
    _run_full(q, k, v, m, b, b, 0.125, what="single block")
    # negative and zero scale
    mask = rand_mask(B, H, n, n, 0.5, seed=11, empty_rows=[(1, 1, 3)])
    _run_full(q, k, v, mask, b, b, -0.3, what="negative scale")
    _run_full(q, k, v, mask, b, b, 0.0, what="zero scale")
    # large score magnitudes: a shared offset on every key (checks max subtraction)
    c = 4.0 * torch.randn(D, generator=torch.Generator().manual_seed(5))
    k2 = (k.float() + c).to(dtype)
    _run_full(q, k2, v, mask, b, b, 0.125, what="shifted keys")


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("bk", [128, 64])
def test_long_rows_every_config(bk, D):
    """Rows with more than 64 active key blocks (kernels that hold the row's list
    64 entries at a time must reload it): block-causal, S = 16384, every config
    of both head dims (the row-pair configs included), on sampled rows from the
    first and the last query blocks."""
    ensure_built()
    B, H, S, bq = 1, 1, 16384, 128
    q, k, v = rand_qkv(B, H, S, D, torch.bfloat16, seed=51)
    n_q, n_k = S // bq, S // bk
    qi = torch.arange(n_q)[:, None]
    kj = torch.arange(n_k)[None, :]
    mask = (kj * bk < (qi + 1) * bq).to(torch.uint8).expand(B, H, n_q, n_k).contiguous()
    assert int(mask[0, 0, -1].sum()) > 64
    rows = np.concatenate([np.arange(0, 256, 37), np.arange(S - 1024, S, 61), [S - 1]]).astype(np.int64)
    ro, rl = oracle.fwd_rows(q, k, v, mask, bq, bk, 0.088, rows)
    qd, kd, vd, md = q.cuda(), k.cuda(), v.cuda(), mask.cuda()
    idx = torch.as_tensor(rows, device="cuda")
    for cfg in bs.list_configs(torch.bfloat16, D, bq, bk):
        say("long rows", D, bk, cfg)
        out, lse = bs.fwd(qd, kd, vd, md, bq, bk, 0.088, config=cfg)
        torch.cuda.synchronize()
        compare(out.reshape(-1, D)[idx], lse.reshape(-1)[idx], ro, rl, "bf16", "long rows %s" % (cfg,))


@pytest.mark.parametrize("D", [128, 64])
def test_row_pair_edge_cases(D):
    """Row-pair configs (tile_q 256): both rows of a pair empty, one empty, an odd
    number of query blocks (last pair has one row), lists that differ, every
    pair config; whole output against the oracle, and fwd_compacted agrees."""
    ensure_built()
    B, H, S, b = 1, 2, 640, 128
    q, k, v = rand_qkv(B, H, S, D, torch.bfloat16, seed=61)
    n = S // b
    mask = torch.zeros(B, H, n, n, dtype=torch.uint8)
    mask[0, 0, 2, :] = 1          # pair 0 of head 0: both rows empty; pair 1: row 3 empty
    mask[0, 0, 4, 1] = 1          # pair 2: one row (n_q odd), one block
    g = torch.Generator().manual_seed(62)
    mask[0, 1] = (torch.rand(n, n, generator=g) < 0.4).to(torch.uint8)
    mask[0, 1, 1] = 0
    mask[0, 1, 1, 4] = 1          # rows 0/1 of head 1: very different lists
    ro, rl = oracle.fwd(q, k, v, mask, b, b, 0.1)
    qd, kd, vd, md = q.cuda(), k.cuda(), v.cuda(), mask.cuda()
    rp, ci = bs.compact_mask(md)
    cfgs = [c for c in bs.list_configs(torch.bfloat16, D, b, b) if c.tile_q == 256]
    assert cfgs
    for cfg in cfgs:
        say("row pairs", D, cfg)
        out, lse = bs.fwd(qd, kd, vd, md, b, b, 0.1, config=cfg)
        o2, l2 = bs.fwd_compacted(qd, kd, vd, rp, ci, b, b, 0.1, config=cfg)
        torch.cuda.synchronize()
        compare(out, lse, ro, rl, "bf16", "pairs %s" % (cfg,))
        assert torch.equal(out, o2) and torch.equal(lse, l2)


def test_compacted_matches_fwd():
    ensure_built()
    B, H, S, D, b = 1, 4, 512, 128, 128
    q, k, v = rand_qkv(B, H, S, D, torch.bfloat16, seed=21)
    mask = rand_mask(B, H, S // b, S // b, 0.5, seed=22)
    qd, kd, vd, md = q.cuda(), k.cuda(), v.cuda(), mask.cuda()
    o1, l1 = bs.fwd(qd, kd, vd, md, b, b, 0.09)
    rp, ci = bs.compact_mask(md)
    o2, l2 = bs.fwd_compacted(qd, kd, vd, rp, ci, b, b, 0.09)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.bfloat16, 64),
                                     (torch.float32, 64)])
def test_planned_matches_fwd(dtype, D):
    """One plan, every built tile config: bsattn_fwd_planned equals bsattn_fwd_config
    bit for bit, and the plan stays valid for new q/k/v of the same mask."""
    ensure_built()
    B, H, S, b = 2, 3, 640, 128
    mask = rand_mask(B, H, S // b, S // b, 0.4, seed=41, empty_rows=[(1, 2, 0)])
    md = mask.cuda()
    ws = bs.plan(md, S, b, b)
    for seed in (42, 43):
        q, k, v = rand_qkv(B, H, S, D, dtype, seed=seed)
        qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        for cfg in bs.list_configs(dtype, D, b, b):
            say("planned", dtype, D, seed, cfg)
            o1, l1 = bs.fwd(qd, kd, vd, md, b, b, 0.11, config=cfg)
            o2, l2 = bs.fwd_planned(qd, kd, vd, ws, b, b, 0.11, config=cfg)
            torch.cuda.synchronize()
            assert torch.equal(o1, o2) and torch.equal(l1, l2), cfg
        orf, lrf = oracle.fwd(q, k, v, mask, b, b, 0.11)
        compare(o2, l2, orf, lrf, dkey(q), what="planned")


def test_deterministic():
    ensure_built()
    w = W.WORKLOADS["sparse_bf16"]
    B, H, S = 1, 4, 4096
    q, k, v = rand_qkv(B, H, S, 128, torch.bfloat16, seed=31)
    mask = W.mask_window_global_random(B, H, S // 128, S // 128, seed=7)
    qd, kd, vd, md = q.cuda(), k.cuda(), v.cuda(), mask.cuda()
    o1, l1 = bs.fwd(qd, kd, vd, md, 128, 128, w.scale)
    o2, l2 = bs.fwd(qd, kd, vd, md, 128, 128, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)



@pytest.mark.parametrize("D,bk,pair", [(128, 128, (256, 128, 8, 2)), (128, 64, (256, 64, 8, 2)),
                                       (64, 64, (256, 64, 8, 2)), (64, 128, (256, 64, 8, 2))])
def test_builtin_default_is_row_pair(D, bk, pair):
    """With no config, no BSATTN_CONFIG and no tuning entry for the shape, a bf16 call
    with 128-row mask blocks runs the row-pair kernel: bit for bit the output of the
    named pair config (shapes chosen to match no tuning entry of other tests)."""
    ensure_built()
    B, H, S = 1, 3, 896
    q, k, v = (t.cuda() for t in rand_qkv(B, H, S, D, torch.bfloat16, seed=D + bk))
    mask = rand_mask(B, H, S // 128, S // bk, 0.6, seed=D + bk, diag=True).cuda()
    o1, l1 = bs.fwd(q, k, v, mask, 128, bk, 1.0 / np.sqrt(D))
    o2, l2 = bs.fwd(q, k, v, mask, 128, bk, 1.0 / np.sqrt(D), config=pair)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_largest_head(dtype):
    """The largest head the boundary takes for D = 128: S = 2^22 - 128, so S*D*4 =
    2^31 - 65536 sits just under the 32-bit byte range of the buffer one head is read
    through (fp32: K and V of a head span it almost whole).  32767 key blocks per row,
    1 GiB of mask: the diagonal, the last key block in every row (the highest K/V
    addresses), two random blocks per row and one empty row; sampled rows, the first
    and last query rows among them, against the oracle."""
    ensure_built()
    B, H, D, b = 1, 1, 128, 128
    S = (1 << 22) - 128
    n = S // b
    assert S * D * 4 < (1 << 31) and (S + 128) * D * 4 == 1 << 31
    say("largest head", dtype, (B, H, S, D))
    q, k, v = rand_qkv(B, H, S, D, dtype, seed=73)
    g = torch.Generator().manual_seed(73)
    mask = torch.zeros(B, H, n, n, dtype=torch.uint8)
    i = torch.arange(n)
    mask[0, 0, i, i] = 1
    mask[0, 0, :, n - 1] = 1
    for _ in range(2):
        mask[0, 0, i, torch.randint(0, n, (n,), generator=g)] = 1
    mask[0, 0, 5] = 0
    qd, kd, vd, md = q.cuda(), k.cuda(), v.cuda(), mask.cuda()
    out, lse = bs.fwd(qd, kd, vd, md, b, b)
    torch.cuda.synchronize()
    rows = np.union1d(W.sample_rows(B, H, S, b, 24, mask=mask), [5 * b, 5 * b + 77, S - 1])
    ro, rl = oracle.fwd_rows(q, k, v, mask, b, b, 1.0 / np.sqrt(D), rows)
    go = out.reshape(-1, D)[torch.as_tensor(rows, device=out.device)]
    gl = lse.reshape(-1)[torch.as_tensor(rows, device=lse.device)]
    kind = "bf16" if dtype == torch.bfloat16 else "f32"
    say("  stats", compare(go, gl, ro, rl, kind, "largest head %s" % kind))
    assert torch.all(out[0, 0, 5 * b:6 * b] == 0) and torch.all(torch.isinf(lse[0, 0, 5 * b:6 * b]))


def test_rows_past_the_pair_limit():
    """Rows of more than 2048 key blocks (S = 262272, 128-key blocks, 2049 per row):
    the row-pair configs refuse the shape, the call with no config falls back to a
    plain config, and sampled rows match the oracle."""
    ensure_built()
    B, H, S, D, b = 1, 1, 2049 * 128, 64, 128
    n = S // b
    q, k, v = rand_qkv(B, H, S, D, torch.bfloat16, seed=71)
    g = torch.Generator().manual_seed(71)
    mask = (torch.rand(B, H, n, n, generator=g) < 0.002).to(torch.uint8)
    mask[..., torch.arange(n), torch.arange(n)] = 1  # the diagonal
    mask[..., :, n - 1] = 1                          # the last key block in every row
    qd, kd, vd, md = q.cuda(), k.cuda(), v.cuda(), mask.cuda()
    with pytest.raises(bs.BsattnError):
        bs.fwd(qd, kd, vd, md, b, b, config=(256, 64, 8, 2))
    out, lse = bs.fwd(qd, kd, vd, md, b, b)
    torch.cuda.synchronize()
    rows = W.sample_rows(B, H, S, b, 32, mask=mask)
    ro, rl = oracle.fwd_rows(q, k, v, mask, b, b, 1.0 / np.sqrt(D), rows)
    go = out.reshape(-1, D)[torch.as_tensor(rows, device=out.device)]
    gl = lse.reshape(-1)[torch.as_tensor(rows, device=lse.device)]
    say("  stats", compare(go, gl, ro, rl, "bf16", "rows past the pair limit"))
