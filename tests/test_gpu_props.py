"""Properties of the GPU forward that hold at any size (invariants of masked
softmax attention), and the autotuner."""
import json
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import bs, compare, ensure_built, rand_mask, rand_qkv, say

pytestmark = pytest.mark.gpu


def _fwd(q, k, v, mask, b, scale, **kw):
    ensure_built()
    out, lse = bs.fwd(q.cuda(), k.cuda(), v.cuda(), mask.cuda(), b, b, scale, **kw)
    torch.cuda.synchronize()
    return out.float().cpu(), lse.cpu()


def _visible(mask, b):
    return mask.repeat_interleave(b, 2).repeat_interleave(b, 3).bool()  # [B,H,S,S]


@pytest.mark.parametrize("D", [64, 128])
def test_key_permutation_within_blocks(D):
    B, H, S, b = 1, 4, 512, 128
    q, k, v = rand_qkv(B, H, S, D, torch.bfloat16, seed=41)
    mask = rand_mask(B, H, S // b, S // b, 0.5, seed=42)
    g = torch.Generator().manual_seed(43)
    perm = torch.cat([torch.randperm(b, generator=g) + j * b for j in range(S // b)])
    say("key permutation", D)
    o1, l1 = _fwd(q, k, v, mask, b, 1 / math.sqrt(D))
    o2, l2 = _fwd(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), mask, b, 1 / math.sqrt(D))
    assert float((o1 - o2).abs().max()) <= 1e-2
    assert float((l1 - l2).abs().max()) <= 1e-3


def test_constant_v():
    B, H, S, D, b = 2, 2, 512, 128, 64
    q, k, _ = rand_qkv(B, H, S, D, torch.bfloat16, seed=51)
    v = torch.full((B, H, S, D), 0.75, dtype=torch.bfloat16)
    mask = rand_mask(B, H, S // b, S // b, 0.4, seed=52, empty_rows=[(1, 1, 2)])
    say("constant V")
    out, lse = _fwd(q, k, v, mask, b, 0.2)
    vis = _visible(mask, b).any(-1)
    assert float((out[vis] - 0.75).abs().max()) <= 0.75 * 2 ** -7
    assert bool((out[~vis] == 0).all()) and bool(torch.isneginf(lse[~vis]).all())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_zero_query_closed_form(dtype):
    # Q = 0: every visible key has weight 1/count, so out = mean of visible V rows
    # and lse = ln(count) exactly.
    B, H, S, D, b = 1, 3, 384, 64, 64
    _, k, v = rand_qkv(B, H, S, D, dtype, seed=61)
    q = torch.zeros(B, H, S, D, dtype=dtype)
    mask = rand_mask(B, H, S // b, S // b, 0.5, seed=62, empty_rows=[(0, 2, 1)])
    say("zero query", dtype)
    out, lse = _fwd(q, k, v, mask, b, 0.7)
    vis = _visible(mask, b).double()
    cnt = vis.sum(-1)
    want = (vis @ v.double()) / cnt.clamp(min=1)[..., None]
    want_lse = torch.where(cnt > 0, cnt.clamp(min=1).log(), torch.full_like(cnt, -math.inf))
    tol = 1e-2 if dtype == torch.bfloat16 else 1e-5
    assert float((out.double() - want).abs().max()) <= tol
    fin = cnt > 0
    assert float((lse.double()[fin] - want_lse[fin]).abs().max()) <= 1e-5
    assert bool(torch.isneginf(lse[~fin]).all())


def test_shift_invariance():
    # K values on a 1/16 grid in [-2, 2) plus a shift of 4 stay exact in bf16, so
    # out(K + c) = out(K) and lse(K + c) = lse(K) + scale * q.c hold up to GPU rounding.
    B, H, S, D, b = 1, 2, 512, 128, 128
    g = torch.Generator().manual_seed(71)
    q = (torch.randint(-16, 16, (B, H, S, D), generator=g) / 16).to(torch.bfloat16)
    k = (torch.randint(-32, 32, (B, H, S, D), generator=g) / 16).to(torch.bfloat16)
    v = torch.randn(B, H, S, D, generator=g).to(torch.bfloat16)
    c = torch.full((D,), 4.0)
    k2 = (k.float() + c).to(torch.bfloat16)
    assert torch.equal(k2.float() - c, k.float())  # the shift is exact
    mask = rand_mask(B, H, S // b, S // b, 0.6, seed=72)
    scale = 0.0625
    say("shift")
    o1, l1 = _fwd(q, k, v, mask, b, scale)
    o2, l2 = _fwd(q, k2, v, mask, b, scale)
    assert float((o1 - o2).abs().max()) <= 1e-2
    dl = scale * (q.float() @ c)
    assert float((l2 - (l1 + dl)).abs().max()) <= 2e-3


def test_autotune_and_cache(tmp_path):
    ensure_built()
    B, H, S, D, b = 1, 4, 1024, 128, 128
    q, k, v = rand_qkv(B, H, S, D, torch.bfloat16, seed=81)
    mask = rand_mask(B, H, S // b, S // b, 0.5, seed=82)
    qd, kd, vd, md = q.cuda(), k.cuda(), v.cuda(), mask.cuda()
    path = tmp_path / "tune.json"
    say("autotune")
    best, rows = bs.autotune(qd, kd, vd, md, b, b, 0.09, warmup=1, iters=3, cache_path=str(path))
    cfgs = [c.as_tuple() for c in bs.list_configs(torch.bfloat16, D, b, b)]
    assert best.as_tuple() in cfgs and len(rows) == len(cfgs)
    assert rows[0].config == best.as_tuple()
    assert all(rows[i].t_mean_s <= rows[i + 1].t_mean_s for i in range(len(rows) - 1))
    assert all(r.t_min_s <= r.t_mean_s for r in rows)
    entries = json.load(open(path))["entries"]
    assert any(e["S"] == S and e["BH"] == B * H and
               (e["tile_q"], e["tile_k"], e["waves"], e["stages"]) == best.as_tuple()
               for e in entries)
    # every timed config gives the oracle's result, and the cached choice is used
    ro, rl = oracle.fwd(q, k, v, mask, b, b, 0.09)
    for cfg in cfgs:
        out, lse = bs.fwd(qd, kd, vd, md, b, b, 0.09, config=cfg)
        torch.cuda.synchronize()
        compare(out, lse, ro, rl, "bf16", str(cfg))
    bs.clear_tune_cache()
    bs.load_tune_cache(str(path))
    out, lse = bs.fwd(qd, kd, vd, md, b, b, 0.09)
    torch.cuda.synchronize()
    compare(out, lse, ro, rl, "bf16", "cached")
    bs.clear_tune_cache()


def test_autotune_two_masks_one_shape(tmp_path):
    """A dense and a sparse mask of one shape tune into separate cache entries
    (the key holds the mask statistic), each found again by its block count."""
    ensure_built()
    B, H, S, D, b = 1, 4, 2048, 128, 128
    q, k, v = rand_qkv(B, H, S, D, torch.bfloat16, seed=83)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    n = S // b
    dense = torch.ones(B, H, n, n, dtype=torch.uint8)
    sparse = torch.zeros(B, H, n, n, dtype=torch.uint8)
    idx = torch.arange(n)
    sparse[:, :, idx, idx] = 1                      # one block per row
    path = tmp_path / "tune.json"
    bs.clear_tune_cache()
    picks = {}
    for name, m in (("dense", dense), ("sparse", sparse)):
        say("autotune", name)
        best, _ = bs.autotune(qd, kd, vd, m.cuda(), b, b, 0.09, warmup=1, iters=2, cache_path=str(path))
        picks[name] = (int(m.sum()), best.as_tuple())
    entries = [e for e in json.load(open(path))["entries"] if e["S"] == S and e["BH"] == B * H]
    buckets = sorted(e["mask_bucket"] for e in entries)
    assert buckets == [0, 8], buckets                # mean 1 and 16 blocks per row
    for name, (nnz, cfg) in picks.items():
        assert bs.tune_lookup(torch.bfloat16, D, B, H, S, b, b, nnz).as_tuple() == cfg, name
    assert bs.tune_lookup(torch.bfloat16, D, B, H, S, b, b, -1).as_tuple() == picks["dense"][1]
    bs.clear_tune_cache()
