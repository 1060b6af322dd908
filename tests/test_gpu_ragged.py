"""Ragged dot on the GPU (bsattn_ragged_dot) against the fp64 oracle on identical
seeded bf16 inputs.

Tolerance, derived from the arithmetic: products of bf16 values are exact in
fp32; fp32 accumulation of K products in any order errs by at most
K * 2^-24 * sum_k |x_k w_k|; a bf16 output adds a rounding of at most 2^-8
|out| (half an ulp of 8 significant bits).  Every element is checked against
that bound, and the mean error must be well below it."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import bs, ensure_built, say

pytestmark = pytest.mark.gpu


def _inputs(M, K, N, G, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16)
    w = torch.randn(G, K, N, generator=g).to(torch.bfloat16)
    return x, w


def _check(x, w, sizes, out_dtype, what, rows=None):
    """GPU result for sizes (as given, may hold negatives / overflow) against the
    oracle on the same sizes (its reading: a negative size is 0 rows, a group
    takes at most the rows that remain)."""
    ensure_built()
    M, K = x.shape
    G, _, N = w.shape
    say("ragged", what, (M, K, N, G), out_dtype)
    out = bs.ragged_dot(x.cuda(), w.cuda(), torch.as_tensor(sizes, dtype=torch.int32).cuda(),
                        out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref = oracle.ragged_dot(x, w, sizes)
    # sum_k |x_k w_k| per element for the bound: the oracle on |x| and |w|
    mag = oracle.ragged_dot(x.double().abs(), w.double().abs(), sizes)
    got = out.double().cpu().numpy()
    if rows is not None:
        got, ref, mag = got[rows], ref[rows], mag[rows]
    bound = K * 2.0 ** -24 * mag + (2.0 ** -8 * np.abs(ref) if out_dtype == torch.bfloat16 else 0.0)
    err = np.abs(got - ref)
    assert np.all(err <= bound + 1e-30), (what, float((err - bound).max()))
    tail = ref == 0.0
    assert np.all(got[np.all(tail, axis=1)] == 0.0), (what, "rows of no group must be 0")
    # the accumulation error is far below its worst case; a bf16 output's rounding
    # error is spread evenly up to half an ulp (between 2^-9 and 2^-8 of |out|), so
    # its mean ratio to the 2^-8 |out| bound is about 0.35
    rel = err[bound > 0] / bound[bound > 0]
    assert rel.mean() < (0.25 if out_dtype == torch.float32 else 0.5), (what, float(rel.mean()))
    return float(rel.max())


CASES = [
    # M, K, N, G, sizes
    (128, 64, 128, 1, [128]),                       # one tile, one group
    (300, 128, 256, 3, [100, 0, 150]),              # an empty group, a zero tail (50 rows)
    (257, 64, 128, 5, [1, 2, 3, 4, 247]),           # many groups in one tile, ragged M
    (512, 192, 384, 4, [130, 126, 129, 127]),       # every tile split between groups
    (200, 64, 128, 3, [-5, 120, 500]),              # a negative size (0) and an overflow (clamped)
    (1024, 256, 128, 2, [0, 1024]),
    (700, 128, 512, 3, [300, 250, 100]),            # 256-column tiles, rows past M in the last tile
    # more (item, 256-column tile) pairs than CUs: full rounds of 256 x 256 tiles and
    # the partial last round as 128 x 128 tiles (an empty group, a 920-row zero tail)
    (17920, 64, 1024, 5, [5000, 3000, 0, 6000, 3000]),
    (8192, 64, 2048, 1, [8192]),                    # exactly one full round on 256 CUs
    # 304 tiles of four 64-deep k-steps: a whole round and a partial one; an empty
    # group, a 300-row zero tail
    (9000, 256, 2048, 4, [3000, 2500, 0, 3200]),
    (5000, 512, 1024, 3, [1000, 2000, 1900]),      # eight k-steps per tile, a zero tail
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:4])))
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_ragged_small(case, out_dtype):
    M, K, N, G, sizes = case
    x, w = _inputs(M, K, N, G, seed=M + K + N)
    _check(x, w, sizes, out_dtype, str(case))


def test_ragged_two_calls_reuse_workspace():
    """Two calls in a row on one workspace with different group sizes."""
    ensure_built()
    x, w = _inputs(384, 128, 256, 3, seed=5)
    ws = torch.empty(4096, dtype=torch.uint8, device="cuda")
    for sizes in ([200, 100, 84], [10, 300, 0]):
        out = bs.ragged_dot(x.cuda(), w.cuda(), torch.tensor(sizes, dtype=torch.int32).cuda(),
                            out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.ragged_dot(x, w, sizes)
        assert np.allclose(out.double().cpu().numpy(), ref, rtol=0, atol=1e-2)


def test_ragged_workload_sampled_rows():
    """The full-size workload (M 32768, K 2048, N 2048, 8 experts) on sampled rows,
    in the launch configuration bench.py times."""
    wl = W.RAGGED_WORKLOADS["ragged_bf16"]
    x, w, sizes = W.make_ragged(wl)
    g = np.random.default_rng(11)
    starts = np.concatenate([[0], np.cumsum(sizes.numpy())])
    rows = set(int(r) for r in g.integers(0, wl.M, 24))
    rows |= {int(s) for s in starts[:-1]} | {int(s) - 1 for s in starts[1:]}  # group edges
    rows = np.array(sorted(r for r in rows if 0 <= r < wl.M))
    ensure_built()
    out = bs.ragged_dot(x.cuda(), w.cuda(), sizes.cuda())
    torch.cuda.synchronize()
    # oracle on the sampled rows only: each row against its own expert
    grp = np.searchsorted(starts, rows, side="right") - 1
    ref = np.stack([x[r].double().numpy() @ w[gi].double().numpy() for r, gi in zip(rows, grp)])
    mag = np.stack([np.abs(x[r].double().numpy()) @ np.abs(w[gi].double().numpy()) for r, gi in zip(rows, grp)])
    got = out.double().cpu().numpy()[rows]
    bound = wl.K * 2.0 ** -24 * mag + 2.0 ** -8 * np.abs(ref)
    assert np.all(np.abs(got - ref) <= bound)


@pytest.mark.timeout(600)
def test_ragged_workload_full():
    """The full-size workload (M 32768, K 2048, N 2048, 8 experts) in the launch
    configuration bench.py times: every output element against the oracle's full
    ragged dot, each held to its bound (the magnitude sums for the bound by a
    float64 matrix product per group of |x| and |w|)."""
    import time
    wl = W.RAGGED_WORKLOADS["ragged_bf16"]
    x, w, sizes = W.make_ragged(wl)
    ensure_built()
    say("ragged workload, full output", (wl.M, wl.K, wl.N, wl.G))
    out = bs.ragged_dot(x.cuda(), w.cuda(), sizes.cuda())
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    say("oracle ragged dot, full output on", oracle.max_threads(), "threads ...")
    t0 = time.perf_counter()
    ref = oracle.ragged_dot(x, w, sizes)
    say("oracle done in %.1f s" % (time.perf_counter() - t0))
    starts = np.concatenate([[0], np.cumsum(sizes.numpy())])
    assert starts[-1] == wl.M
    ax = np.abs(x.double().numpy())
    worst = 0.0
    for gi in range(wl.G):
        r0, r1 = int(starts[gi]), int(starts[gi + 1])
        mag = ax[r0:r1] @ np.abs(w[gi].double().numpy())
        bound = wl.K * 2.0 ** -24 * mag + 2.0 ** -8 * np.abs(ref[r0:r1])
        err = np.abs(got[r0:r1] - ref[r0:r1])
        assert np.all(err <= bound), ("group", gi, float((err - bound).max()))
        rel = err[bound > 0] / bound[bound > 0]
        assert rel.mean() < 0.5, ("group", gi, float(rel.mean()))
        worst = max(worst, float(err.max()))
    say("  max err over all elements", worst)


def test_ragged_planned_equals_one_shot():
    """bsattn_ragged_plan + bsattn_ragged_dot_planned gives bit for bit the result
    of bsattn_ragged_dot (the same plan and product kernels)."""
    ensure_built()
    x, w = _inputs(700, 128, 256, 4, seed=17)
    sizes = torch.tensor([300, 0, 250, 90], dtype=torch.int32).cuda()  # 60-row zero tail
    a = bs.ragged_dot(x.cuda(), w.cuda(), sizes)
    ws = bs.ragged_plan(sizes, 700)
    b = bs.ragged_dot_planned(x.cuda(), w.cuda(), ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.all(b[640:] == 0)


@pytest.mark.timeout(600)
def test_ragged_largest_expert():
    """One expert's rhs just under the 2 GiB one buffer addresses (K 2048, N 524160:
    K*N*2 = 2^31 - 2^19), two experts, so the second starts past byte 2^31 of rhs;
    M 512 with 62 rows in no group.  Sampled rows of each group against the oracle
    (the same function on the sampled rows alone: the product is row by row), each
    element held to its bound; the rows in no group exactly 0."""
    ensure_built()
    M, K, N, G = 512, 2048, 524160, 2
    assert K * N * 2 < (1 << 31) and (1 << 31) - K * N * 2 == 1 << 19
    say("ragged largest expert", (M, K, N, G))
    gen = torch.Generator().manual_seed(77)
    x = torch.randn(M, K, generator=gen).to(torch.bfloat16)
    gd = torch.Generator(device="cuda").manual_seed(77)
    wd = torch.randn(G, K, N, generator=gd, device="cuda").to(torch.bfloat16)
    sizes = torch.tensor([200, 250], dtype=torch.int32)
    out = bs.ragged_dot(x.cuda(), wd, sizes.cuda())
    torch.cuda.synchronize()
    assert torch.all(out[450:] == 0)
    w = wd.cpu()
    del wd
    picks = [[0, 1, 117, 198, 199], [200, 201, 333, 448, 449]]
    rows = np.array(picks[0] + picks[1])
    sub_sizes = torch.tensor([len(picks[0]), len(picks[1])], dtype=torch.int32)
    xs = x[torch.as_tensor(rows)]
    say("  oracle on", len(rows), "rows,", oracle.max_threads(), "threads")
    ref = oracle.ragged_dot(xs, w, sub_sizes)
    mag = oracle.ragged_dot(xs.abs(), w.abs(), sub_sizes)  # |bf16| is exact
    got = out[torch.as_tensor(rows, device="cuda")].double().cpu().numpy()
    bound = K * 2.0 ** -24 * mag + 2.0 ** -8 * np.abs(ref)
    err = np.abs(got - ref)
    assert np.all(err <= bound), float((err - bound).max())
    rel = err[bound > 0] / bound[bound > 0]
    assert rel.mean() < 0.5, float(rel.mean())
    say("  max err", float(err.max()))
