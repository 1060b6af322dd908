"""bsattn_fwd_noalloc (the forward whose plan lives in the library's fixed
device array) against bsattn_fwd_config with a caller workspace: the same
kernels on the same plan, so out and lse must agree bit for bit, and both
against the fp64 oracle at the bf16 / fp32 tolerances.  Two calls in a row,
the second on a smaller input (its plan overwrites a part of the first's), then
the first shape again."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import bs, compare, dkey, ensure_built, rand_mask, rand_qkv, say

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, S, D, block_q, block_k, dtype, p, config
    (2, 4, 4096, 128, 128, 128, torch.bfloat16, 0.5, (256, 128, 8, 2)),
    (1, 2, 640, 64, 64, 128, torch.bfloat16, 0.4, None),
    (1, 2, 256, 64, 64, 64, torch.float32, 0.5, None),
    (2, 4, 4096, 128, 128, 128, torch.bfloat16, 0.5, (256, 128, 8, 2)),
]


def test_no_alloc_equals_workspace_forward():
    ensure_built()
    assert bs.noalloc_max_bytes() == 16 << 20
    for i, (B, H, S, D, bq, bk, dt, p, cfg) in enumerate(CASES):
        say("no-alloc call", i, (B, H, S, D, bq, bk), dt, cfg)
        q, k, v = rand_qkv(B, H, S, D, dt, seed=100 + i)
        mask = rand_mask(B, H, S // bq, S // bk, p, seed=200 + i, empty_rows=[(0, 1, 2)])
        qd, kd, vd, md = q.cuda(), k.cuda(), v.cuda(), mask.cuda()
        out = torch.empty_like(qd)
        lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
        bs.fwd_noalloc(qd, kd, vd, md, bq, bk, 1.0 / np.sqrt(D), out, lse, config=cfg)
        o2, l2 = bs.fwd(qd, kd, vd, md, bq, bk, 1.0 / np.sqrt(D), config=cfg)
        torch.cuda.synchronize()
        assert torch.equal(out, o2) and torch.equal(lse, l2), i
        ro, rl = oracle.fwd(q, k, v, mask, bq, bk, 1.0 / np.sqrt(D))
        say("  ", compare(out, lse, ro, rl, dkey(q), "no-alloc %d" % i))


def test_no_alloc_refuses_a_plan_beyond_the_array():
    """A mask whose plan needs more than the fixed array is refused on the host
    (BSATTN_ERR_WORKSPACE) before any device work; the outputs stay untouched."""
    ensure_built()
    B, H, S, D, b = 1, 64, 65536, 64, 128   # 64 heads x 512 x 512 blocks: 64 MiB of lists
    assert bs.workspace_size(B, H, S, b, b) > bs.noalloc_max_bytes()
    q = torch.zeros(B, H, S, D, dtype=torch.bfloat16, device="cuda")
    mask = torch.zeros(B, H, S // b, S // b, dtype=torch.uint8, device="cuda")
    out = torch.full_like(q, 7.0)
    lse = torch.full((B, H, S), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(bs.BsattnError) as e:
        bs.fwd_noalloc(q, q, q, mask, b, b, 0.125, out, lse)
    assert e.value.status == 5
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())
