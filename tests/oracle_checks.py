"""Pins of the fp64 oracle against things other than itself.

Each check takes the oracle's Python API (a module or object with fwd, fwd_rows,
probs, compact) so the same checks run on the real oracle (test_oracle_pins.py)
and on deliberately broken copies of it (test_oracle_mutants.py).

What pins what:
  hand_example      hand-derived values of a 4-token example (tests/golden)
  brute_force       dense literal -inf softmax in NumPy + scipy logsumexp
  sdpa_dense        torch scaled_dot_product_attention (fp64, CPU) for an all-ones mask
  sdpa_block_causal torch SDPA with the expanded lower-triangular block mask
  block_diagonal    block-diagonal mask == independent dense attention per block
  probs_sum         softmax weights are >= 0, zero where masked, rows sum to 1
  constant_v        V == c gives out == c on every non-empty row
  zero_query        Q == 0 (or scale == 0): out = mean of the visible V rows,
                    lse = ln(number of visible keys)
  empty_rows        a row with no active block gives out == 0 exactly, lse == -inf
  linearity         out(a V1 + b V2) == a out(V1) + b out(V2)
  key_permutation   permuting keys (with their V rows) inside an active block
                    changes neither out nor lse
  shift             K + 1 c^T leaves out unchanged and adds scale*(q.c) to lse;
                    with a large c it also checks the max subtraction
  rows_match_full   the selected-rows entry point equals the full forward
  bf16_widening     bf16 inputs give the same result as their exact fp64 values
  fp8_widening      every e4m3 byte (one key per query, so out = v) equals torch's
                    float8_e4m3fn -> float64 conversion; NaN codes give NaN
  compact_brute     CSR compaction equals np.nonzero per row
Element-level masks (block states 0/1/partial + bit tiles):
  elem_brute        dense literal -inf softmax over the expanded element mask
  elem_tiles_all_set / elem_tiles_all_clear
                    partial blocks whose tiles are all ones (zeros) equal the
                    block-level oracle with those blocks active (inactive)
  elem_token_causal torch SDPA with is_causal (fp64, CPU): block causal states
                    with one lower-triangular tile on the diagonal blocks
  elem_empty_row    a query row whose only active block is partial with that
                    row's bits all clear gives out == 0, lse == -inf
  elem_rows_match   the selected-rows entry point equals the full forward
Ragged dot (expert matrices stacked on the right, rows assigned in order):
  ragged_hand       a 4-row example worked out by hand (expert 1 empty, a tail row)
  ragged_sizes      negative and overflowing group sizes, worked out by hand (tests/golden)
  ragged_one_group  one group of all rows equals numpy matmul
  ragged_permute    reordering the experts with their row blocks reorders the rows
  ragged_linear     out(X, a W1 + b W2) == a out(X, W1) + b out(X, W2)
  ragged_tail       rows past the sum of the sizes are 0; empty groups change nothing
  ragged_bf16       bf16 inputs give the same result as their exact fp64 values
Backward (gradients for an upstream gradient dout):
  bwd_autograd      torch autograd (fp64, CPU) through a dense masked softmax
                    attention built from plain torch ops, empty rows included
  bwd_finite_diff   central differences of sum(dout * out) through the forward
                    oracle, on entries of q, k and v
  bwd_sums          per head: dk summed over keys is 0 (a shift of every key
                    changes no softmax); dv summed over keys is dout summed over
                    the rows that see any key; keys no row sees and rows that see
                    no key get exact zeros
  bwd_constant_v    V == c gives dq == dk == 0
  bwd_linear_dout   the gradients are linear in dout
  bwd_sample_match  the sampled entry point equals the full backward
"""
import json
import math
import os

import numpy as np
import torch

from brute import brute_compact, brute_fwd, brute_fwd_full, expand_elem, expand_mask

HERE = os.path.dirname(os.path.abspath(__file__))
TOL = 1e-12


def _rand(shape, seed, dtype=torch.float64):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float64).to(dtype)


def _mask(B, H, nq, nk, p, seed, empty_rows=()):
    g = torch.Generator().manual_seed(seed)
    m = (torch.rand(B, H, nq, nk, generator=g) < p).to(torch.uint8)
    for (b, h, i) in empty_rows:
        m[b, h, i, :] = 0
    return m


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    fin_a, fin_b = np.isfinite(a), np.isfinite(b)
    assert np.array_equal(fin_a, fin_b), (what, "finite pattern differs")
    assert np.array_equal(a[~fin_a], b[~fin_b], equal_nan=True), (what, "non-finite values differ")
    if fin_a.any():
        err = np.max(np.abs(a[fin_a] - b[fin_b]))
        scale = max(1.0, float(np.max(np.abs(b[fin_b]))))
        assert err <= tol * scale, (what, float(err))


def hand_example(orc):
    ex = json.load(open(os.path.join(HERE, "golden", "hand_example.json")))
    q = np.array(ex["q"], dtype=np.float64)
    k = np.array(ex["k"], dtype=np.float64)
    v = np.array(ex["v"], dtype=np.float64)
    mask = np.array(ex["mask"], dtype=np.uint8)
    out, lse = orc.fwd(q, k, v, mask, ex["block_q"], ex["block_k"], ex["scale"])
    want_lse = np.array([[[float(x) for x in row] for row in h] for h in ex["lse"]])
    _close(out, np.array(ex["out"]), 1e-12, "out")
    _close(lse, want_lse, 1e-12, "lse")


CASES = [
    # B, H, S, D, block_q, block_k, p, seed, dtype, scale
    (1, 1, 8, 4, 2, 2, 0.6, 1, torch.float64, 0.7),
    (2, 3, 16, 8, 4, 2, 0.5, 2, torch.float64, 0.35),
    (1, 2, 12, 5, 3, 4, 0.5, 3, torch.float32, 1.3),
    (2, 2, 32, 16, 8, 16, 0.5, 4, torch.bfloat16, 0.25),
    (1, 2, 24, 6, 6, 4, 0.4, 5, torch.float64, -0.9),
    (1, 2, 32, 16, 8, 8, 0.5, 6, torch.float8_e4m3fn, 0.3),
]


def brute_force(orc):
    for (B, H, S, D, bq, bk, p, seed, dt, scale) in CASES:
        q = _rand((B, H, S, D), seed, dt)
        k = _rand((B, H, S, D), seed + 100, dt)
        v = _rand((B, H, S, D), seed + 200, dt)
        mask = _mask(B, H, S // bq, S // bk, p, seed, empty_rows=[(0, 0, 1)])
        out, lse = orc.fwd(q, k, v, mask, bq, bk, scale)
        bout, blse, _ = brute_fwd(q, k, v, mask, bq, bk, scale)
        _close(out, bout, TOL, "out %s" % (dt,))
        _close(lse, blse, TOL, "lse %s" % (dt,))


def _sdpa(q, k, v, full, scale):
    return torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=torch.as_tensor(full), scale=float(np.float32(scale))).numpy()


def sdpa_dense(orc):
    B, H, S, D, bq, bk = 2, 2, 32, 8, 8, 4
    q, k, v = (_rand((B, H, S, D), s) for s in (11, 12, 13))
    mask = torch.ones(B, H, S // bq, S // bk, dtype=torch.uint8)
    out, _ = orc.fwd(q, k, v, mask, bq, bk, 0.3)
    want = _sdpa(q, k, v, np.ones((B, H, S, S), dtype=bool), 0.3)
    _close(out, want, TOL, "dense")


def sdpa_block_causal(orc):
    B, H, S, D, b = 1, 3, 48, 8, 8
    q, k, v = (_rand((B, H, S, D), s) for s in (21, 22, 23))
    n = S // b
    mask = torch.tril(torch.ones(n, n, dtype=torch.uint8)).expand(B, H, n, n).contiguous()
    out, _ = orc.fwd(q, k, v, mask, b, b, 0.4)
    want = _sdpa(q, k, v, expand_mask(mask, b, b), 0.4)
    _close(out, want, TOL, "block causal")


def block_diagonal(orc):
    B, H, S, D, b = 1, 2, 32, 4, 8
    q, k, v = (_rand((B, H, S, D), s) for s in (31, 32, 33))
    n = S // b
    mask = torch.eye(n, dtype=torch.uint8).expand(B, H, n, n).contiguous()
    out, _ = orc.fwd(q, k, v, mask, b, b, 0.5)
    for i in range(n):
        sl = slice(i * b, (i + 1) * b)
        want = _sdpa(q[:, :, sl], k[:, :, sl], v[:, :, sl], np.ones((B, H, b, b), bool), 0.5)
        _close(out[:, :, sl], want, TOL, "block %d" % i)


def probs_sum(orc):
    B, H, S, D, bq, bk = 2, 2, 16, 4, 4, 2
    q, k, v = (_rand((B, H, S, D), s) for s in (41, 42, 43))
    mask = _mask(B, H, S // bq, S // bk, 0.5, 44, empty_rows=[(1, 1, 2)])
    P = orc.probs(q, k, v, mask, bq, bk, 0.8)
    full = expand_mask(mask, bq, bk)
    assert np.all(P >= 0.0)
    assert np.all(P[~full] == 0.0)
    sums = P.sum(-1)
    nonempty = full.any(-1)
    assert np.all(np.abs(sums[nonempty] - 1.0) <= 1e-14), float(np.max(np.abs(sums[nonempty] - 1)))
    assert np.all(sums[~nonempty] == 0.0)
    # and the probabilities are the brute force's
    _, _, bp = brute_fwd(q, k, v, mask, bq, bk, 0.8)
    _close(P, bp, TOL, "P")


def constant_v(orc):
    B, H, S, D, bq, bk = 1, 2, 16, 6, 4, 4
    q, k = _rand((B, H, S, D), 51), _rand((B, H, S, D), 52)
    v = torch.full((B, H, S, D), 2.75, dtype=torch.float64)
    mask = _mask(B, H, S // bq, S // bk, 0.5, 53, empty_rows=[(0, 1, 0)])
    out, _ = orc.fwd(q, k, v, mask, bq, bk, 1.1)
    nonempty = expand_mask(mask, bq, bk).any(-1)
    assert np.all(np.abs(out[nonempty] - 2.75) <= 1e-13)
    assert np.all(out[~nonempty] == 0.0)


def zero_query(orc):
    B, H, S, D, bq, bk = 1, 2, 24, 5, 6, 3
    k, v = _rand((B, H, S, D), 61), _rand((B, H, S, D), 62)
    mask = _mask(B, H, S // bq, S // bk, 0.5, 63, empty_rows=[(0, 0, 3)])
    full = expand_mask(mask, bq, bk)
    vv = v.numpy()
    cnt = full.sum(-1)
    want_out = np.where(cnt[..., None] > 0,
                        np.einsum("bhij,bhjd->bhid", full.astype(np.float64), vv)
                        / np.maximum(cnt, 1)[..., None], 0.0)
    want_lse = np.where(cnt > 0, np.log(np.maximum(cnt, 1)), -np.inf)
    # Q == 0 with a nonzero scale, and a random Q with scale == 0
    for q, scale in ((torch.zeros(B, H, S, D, dtype=torch.float64), 0.9),
                     (_rand((B, H, S, D), 64), 0.0)):
        out, lse = orc.fwd(q, k, v, mask, bq, bk, scale)
        _close(out, want_out, 1e-13, "out")
        _close(lse, want_lse, 1e-13, "lse")


def empty_rows(orc):
    B, H, S, D, bq, bk = 1, 2, 16, 4, 4, 4
    q, k, v = (_rand((B, H, S, D), s) for s in (71, 72, 73))
    mask = torch.ones(B, H, S // bq, S // bk, dtype=torch.uint8)
    mask[0, 1, 2, :] = 0
    mask[0, 0, 0, :] = 0
    out, lse = orc.fwd(q, k, v, mask, bq, bk, 0.5)
    for (h, i) in ((1, 2), (0, 0)):
        rows = slice(i * bq, (i + 1) * bq)
        assert np.all(out[0, h, rows] == 0.0)
        assert np.all(np.isneginf(lse[0, h, rows]))
    assert np.all(np.isfinite(lse[0, 0, bq:]))


def linearity(orc):
    B, H, S, D, bq, bk = 1, 1, 16, 4, 4, 2
    q, k, v1, v2 = (_rand((B, H, S, D), s) for s in (81, 82, 83, 84))
    mask = _mask(B, H, S // bq, S // bk, 0.6, 85)
    a, b = 1.5, -0.25
    o1, _ = orc.fwd(q, k, v1, mask, bq, bk, 0.6)
    o2, _ = orc.fwd(q, k, v2, mask, bq, bk, 0.6)
    o3, _ = orc.fwd(q, k, a * v1 + b * v2, mask, bq, bk, 0.6)
    _close(o3, a * o1 + b * o2, 1e-12, "linearity")


def key_permutation(orc):
    B, H, S, D, bq, bk = 1, 2, 16, 4, 4, 4
    q, k, v = (_rand((B, H, S, D), s) for s in (91, 92, 93))
    mask = _mask(B, H, S // bq, S // bk, 0.6, 94)
    out, lse = orc.fwd(q, k, v, mask, bq, bk, 0.7)
    g = torch.Generator().manual_seed(95)
    perm = torch.arange(S)
    for kj in range(S // bk):  # shuffle keys inside every key block
        idx = torch.randperm(bk, generator=g) + kj * bk
        perm[kj * bk:(kj + 1) * bk] = idx
    out2, lse2 = orc.fwd(q, k[:, :, perm], v[:, :, perm], mask, bq, bk, 0.7)
    _close(out2, out, 1e-12, "out")
    _close(lse2, lse, 1e-12, "lse")


def shift(orc):
    B, H, S, D, bq, bk = 1, 2, 16, 4, 4, 4
    q, k, v = (_rand((B, H, S, D), s) for s in (101, 102, 103))
    mask = _mask(B, H, S // bq, S // bk, 0.7, 104)
    scale = 0.5
    out, lse = orc.fwd(q, k, v, mask, bq, bk, scale)
    for mag in (1.0, 5000.0):  # 5000 pushes |score| past the fp64 exp range (~709)
        c = mag * _rand((D,), 105)
        out2, lse2 = orc.fwd(q, k + c, v, mask, bq, bk, scale)
        _close(out2, out, 1e-9, "out shift %g" % mag)
        qc = scale * np.einsum("bhsd,d->bhs", q.numpy(), c.numpy())
        want = np.where(np.isfinite(lse), lse + qc, lse)
        _close(lse2, want, 1e-9, "lse shift %g" % mag)


def rows_match_full(orc):
    B, H, S, D, bq, bk = 2, 2, 16, 8, 4, 8
    q, k, v = (_rand((B, H, S, D), s) for s in (111, 112, 113))
    mask = _mask(B, H, S // bq, S // bk, 0.5, 114, empty_rows=[(1, 0, 1)])
    out, lse = orc.fwd(q, k, v, mask, bq, bk, 0.45)
    rows = np.array([0, 5, 17, 33, 40, 63], dtype=np.int64)
    ro, rl = orc.fwd_rows(q, k, v, mask, bq, bk, 0.45, rows)
    assert np.array_equal(ro, out.reshape(-1, D)[rows])
    assert np.array_equal(rl, lse.reshape(-1)[rows])


def bf16_widening(orc):
    B, H, S, D, bq, bk = 1, 2, 16, 8, 4, 4
    q, k, v = (_rand((B, H, S, D), s, torch.bfloat16) for s in (121, 122, 123))
    mask = _mask(B, H, S // bq, S // bk, 0.6, 124)
    o1, l1 = orc.fwd(q, k, v, mask, bq, bk, 0.3)
    o2, l2 = orc.fwd(q.double(), k.double(), v.double(), mask, bq, bk, 0.3)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def fp8_widening(orc):
    n = 256
    codes = torch.arange(n, dtype=torch.int32).to(torch.uint8).view(1, 1, n, 1)
    v = codes.view(torch.float8_e4m3fn).expand(1, 1, n, 2).contiguous()
    q = torch.zeros(1, 1, n, 2, dtype=torch.float8_e4m3fn)
    mask = torch.eye(n, dtype=torch.uint8).view(1, 1, n, n)  # query r sees key r only
    out, lse = orc.fwd(q, q, v, mask, 1, 1, 1.0)
    want = v.to(torch.float64).numpy()
    _close(out, want, 0.0, "fp8 codes")
    _close(lse, np.zeros((1, 1, n)), 0.0, "lse of one key with score 0")


def compact_brute(orc):
    for (shape, p, seed) in (((1, 2, 4, 4), 0.5, 0), ((2, 3, 5, 70), 0.3, 1),
                             ((1, 1, 3, 129), 0.02, 2), ((2, 2, 4, 8), 0.0, 3),
                             ((1, 2, 3, 64), 1.0, 4)):
        g = torch.Generator().manual_seed(seed)
        m = (torch.rand(*shape, generator=g) < p).to(torch.uint8)
        rp, ci = orc.compact(m)
        brp, bci = brute_compact(m)
        assert np.array_equal(rp, brp) and np.array_equal(ci, bci)
        assert rp[-1] == int(m.sum())
        for r in range(len(rp) - 1):  # strictly ascending within each row
            seg = ci[rp[r]:rp[r + 1]]
            assert np.all(np.diff(seg) > 0)
        rebuilt = np.zeros((len(rp) - 1, shape[-1]), dtype=np.uint8)
        for r in range(len(rp) - 1):
            rebuilt[r, ci[rp[r]:rp[r + 1]]] = 1
        assert np.array_equal(rebuilt.reshape(shape), m.numpy())


def _elem_case(B, H, S, bq, bk, n_tiles, seed, p=(0.3, 0.3, 0.4), density=0.5):
    """Random block states (empty / full / partial with probabilities p) and
    n_tiles random bit tiles of the given density."""
    g = np.random.default_rng(seed)
    st = g.choice(3, size=(B, H, S // bq, S // bk), p=p).astype(np.uint8)
    st[st == 2] = g.choice([2, 7, 255], size=int((st == 2).sum()))  # any value > 1 is partial
    pidx = g.integers(0, n_tiles, size=st.shape).astype(np.int32)
    bits = (g.random((n_tiles, bq, bk)) < density)
    pbits = np.packbits(bits, axis=-1, bitorder="little").view(np.uint32).reshape(n_tiles, bq, bk // 32)
    return st, pidx, pbits


ELEM_CASES = [
    # B, H, S, D, block_q, block_k, n_tiles, seed, dtype, scale
    (1, 2, 64, 8, 16, 32, 3, 31, torch.float64, 0.4),
    (2, 1, 96, 4, 8, 32, 5, 32, torch.float32, -0.7),
    (1, 1, 128, 16, 32, 64, 2, 33, torch.bfloat16, 0.25),
]


def elem_brute(orc):
    for (B, H, S, D, bq, bk, nt, seed, dt, scale) in ELEM_CASES:
        q = _rand((B, H, S, D), seed, dt)
        k = _rand((B, H, S, D), seed + 100, dt)
        v = _rand((B, H, S, D), seed + 200, dt)
        st, pidx, pbits = _elem_case(B, H, S, bq, bk, nt, seed)
        out, lse = orc.fwd_elem(q, k, v, st, pidx, pbits, bq, bk, scale)
        bout, blse, _ = brute_fwd_full(q, k, v, expand_elem(st, pidx, pbits, bq, bk), scale)
        _close(out, bout, TOL, "elem out %s" % (dt,))
        _close(lse, blse, TOL, "elem lse %s" % (dt,))


def _elem_vs_block(orc, fill):
    B, H, S, D, bq, bk = 1, 2, 64, 8, 16, 32
    q, k, v = (_rand((B, H, S, D), s) for s in (41, 42, 43))
    st, pidx, pbits = _elem_case(B, H, S, bq, bk, 2, 44)
    pbits[:] = np.uint32(0xFFFFFFFF) if fill else np.uint32(0)
    out, lse = orc.fwd_elem(q, k, v, st, pidx, pbits, bq, bk, 0.5)
    blk = (st != 0) if fill else (st == 1)
    bout, blse = orc.fwd(q, k, v, blk.astype(np.uint8), bq, bk, 0.5)
    _close(out, bout, 0.0, "elem vs block out")
    _close(lse, blse, 0.0, "elem vs block lse")


def elem_tiles_all_set(orc):
    _elem_vs_block(orc, True)


def elem_tiles_all_clear(orc):
    _elem_vs_block(orc, False)


def elem_token_causal(orc):
    B, H, S, D, b = 1, 2, 96, 8, 32
    q, k, v = (_rand((B, H, S, D), s) for s in (51, 52, 53))
    n = S // b
    st = (np.tril(np.ones((n, n), dtype=np.uint8)) + np.eye(n, dtype=np.uint8))  # 1 below, 2 on
    st = np.broadcast_to(st, (B, H, n, n)).copy()
    pidx = np.zeros((B, H, n, n), dtype=np.int32)
    tri = np.tril(np.ones((b, b), dtype=bool))
    pbits = np.packbits(tri, axis=-1, bitorder="little").view(np.uint32).reshape(1, b, b // 32)
    out, lse = orc.fwd_elem(q, k, v, st, pidx, pbits, b, b, 0.3)
    want = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True,
                                                            scale=float(np.float32(0.3))).numpy()
    _close(out, want, TOL, "token causal")


def elem_empty_row(orc):
    B, H, S, D, bq, bk = 1, 1, 64, 4, 16, 32
    q, k, v = (_rand((B, H, S, D), s) for s in (61, 62, 63))
    st = np.zeros((B, H, S // bq, S // bk), dtype=np.uint8)
    st[0, 0, 1, 1] = 2          # query block 1 sees only key block 1, through tile 0
    st[0, 0, 2, :] = 1          # query block 2 sees everything
    pidx = np.zeros(st.shape, dtype=np.int32)
    bits = np.ones((1, bq, bk), dtype=bool)
    bits[0, 5, :] = False       # query 16 + 5 keeps nothing
    pbits = np.packbits(bits, axis=-1, bitorder="little").view(np.uint32).reshape(1, bq, bk // 32)
    out, lse = orc.fwd_elem(q, k, v, st, pidx, pbits, bq, bk, 0.5)
    assert np.all(out[0, 0, 21] == 0.0) and lse[0, 0, 21] == -np.inf
    assert np.all(np.isfinite(lse[0, 0, 16:21])) and np.all(np.isfinite(lse[0, 0, 32:48]))
    assert np.all(lse[0, 0, :16] == -np.inf) and np.all(out[0, 0, :16] == 0.0)


def elem_rows_match(orc):
    (B, H, S, D, bq, bk, nt, seed, dt, scale) = ELEM_CASES[1]
    q = _rand((B, H, S, D), seed, dt)
    k = _rand((B, H, S, D), seed + 100, dt)
    v = _rand((B, H, S, D), seed + 200, dt)
    st, pidx, pbits = _elem_case(B, H, S, bq, bk, nt, seed)
    out, lse = orc.fwd_elem(q, k, v, st, pidx, pbits, bq, bk, scale)
    rows = np.array([0, 5, 17, 95, 96 + 40, 2 * 96 - 1])
    ro, rl = orc.fwd_rows_elem(q, k, v, st, pidx, pbits, bq, bk, scale, rows)
    _close(ro, out.reshape(-1, D)[rows], 0.0, "rows out")
    _close(rl, lse.reshape(-1)[rows], 0.0, "rows lse")


def ragged_hand(orc):
    # lhs rows (0,1) (2,3) (4,5) (6,7); experts [[0,1],[2,3]], [[4,5],[6,7]],
    # [[8,9],[10,11]]; sizes (1, 0, 2): row 0 uses expert 0: (0*0+1*2, 0*1+1*3) = (2, 3);
    # rows 1, 2 use expert 2: (2*8+3*10, 2*9+3*11) = (46, 51), (4*8+5*10, 4*9+5*11) =
    # (82, 91); row 3 belongs to no group: (0, 0).
    lhs = np.arange(8, dtype=np.float64).reshape(4, 2)
    rhs = np.arange(12, dtype=np.float64).reshape(3, 2, 2)
    out = orc.ragged_dot(lhs, rhs, [1, 0, 2])
    assert np.array_equal(out, np.array([[2, 3], [46, 51], [82, 91], [0, 0]], dtype=np.float64))


def ragged_sizes(orc):
    ex = json.load(open(os.path.join(HERE, "golden", "ragged_sizes.json")))
    lhs = np.array(ex["lhs"], dtype=np.float64)
    rhs = np.array(ex["rhs"], dtype=np.float64)
    for case in ex["cases"]:
        out = orc.ragged_dot(lhs, rhs, case["sizes"])
        assert np.array_equal(out, np.array(case["out"], dtype=np.float64)), case["sizes"]


def _ragged_inputs(M, K, N, G, seed, dt=torch.float64):
    x = _rand((M, K), seed, dt)
    w = _rand((G, K, N), seed + 1, dt)
    return x, w


def ragged_one_group(orc):
    x, w = _ragged_inputs(7, 5, 3, 1, 71)
    out = orc.ragged_dot(x, w, [7])
    _close(out, x.numpy() @ w[0].numpy(), TOL, "one group")


def ragged_permute(orc):
    M, K, N = 9, 4, 3
    x, w = _ragged_inputs(M, K, N, 3, 72)
    sizes = [2, 4, 3]
    out = orc.ragged_dot(x, w, sizes)
    # experts in the order (2, 0, 1), the rows moved with them
    xa = x.numpy()
    blocks = [xa[0:2], xa[2:6], xa[6:9]]
    xp = np.concatenate([blocks[2], blocks[0], blocks[1]])
    wp = w.numpy()[[2, 0, 1]]
    outp = orc.ragged_dot(xp, wp, [3, 2, 4])
    _close(outp, np.concatenate([out[6:9], out[0:2], out[2:6]]), TOL, "permute")


def ragged_linear(orc):
    x, w1 = _ragged_inputs(10, 6, 4, 3, 73)
    _, w2 = _ragged_inputs(10, 6, 4, 3, 74)
    sizes = [3, 3, 4]
    a, b = 0.75, -1.5
    lhs = orc.ragged_dot(x, a * w1 + b * w2, sizes)
    rhs = a * orc.ragged_dot(x, w1, sizes) + b * orc.ragged_dot(x, w2, sizes)
    _close(lhs, rhs, 1e-13, "linear")


def ragged_tail(orc):
    x, w = _ragged_inputs(12, 5, 3, 4, 75)
    out = orc.ragged_dot(x, w, [0, 5, 0, 4])
    assert np.all(out[9:] == 0.0)
    # the same rows through a 2-expert stack without the empty experts
    out2 = orc.ragged_dot(x, w[torch.tensor([1, 3])].contiguous(), [5, 4])
    _close(out, out2, 0.0, "empty groups")


def ragged_bf16(orc):
    x, w = _ragged_inputs(6, 8, 5, 2, 76, torch.bfloat16)
    out = orc.ragged_dot(x, w, [2, 3])
    ref = orc.ragged_dot(x.to(torch.float64), w.to(torch.float64), [2, 3])
    _close(out, ref, 0.0, "bf16 widening")


# ---- backward ----------------------------------------------------------------

BWD_CASES = [
    # B, H, S, D, block_q, block_k, p, seed, dtype, scale
    (1, 2, 12, 4, 3, 4, 0.6, 31, torch.float64, 0.8),
    (2, 1, 16, 8, 4, 2, 0.5, 32, torch.float64, -0.45),
    (1, 2, 32, 16, 8, 16, 0.6, 33, torch.bfloat16, 0.25),
    (1, 1, 24, 6, 6, 4, 0.5, 34, torch.float32, 1.1),
]


def _bwd_case(B, H, S, D, bq, bk, p, seed, dt):
    q = _rand((B, H, S, D), seed, dt)
    k = _rand((B, H, S, D), seed + 100, dt)
    v = _rand((B, H, S, D), seed + 200, dt)
    do = _rand((B, H, S, D), seed + 300, dt)
    mask = _mask(B, H, S // bq, S // bk, p, seed, empty_rows=[(0, 0, 1)])
    return q, k, v, do, mask


def _autograd_grads(q, k, v, do, mask, bq, bk, scale):
    """Plain torch ops in fp64 with autograd: scores, -inf where masked, row
    softmax (rows with no visible key contribute 0), times V."""
    full = torch.as_tensor(expand_mask(mask, bq, bk))
    qq, kk, vv = (t.to(torch.float64).clone().requires_grad_(True) for t in (q, k, v))
    s = float(np.float32(scale)) * torch.matmul(qq, kk.transpose(-1, -2))
    anyk = full.any(dim=-1, keepdim=True)
    s = s.masked_fill(~full, float("-inf")).masked_fill(~anyk, 0.0)
    pr = torch.softmax(s, dim=-1) * anyk
    out = torch.matmul(pr, vv)
    loss = (out * do.to(torch.float64)).sum()
    return [g.numpy() for g in torch.autograd.grad(loss, (qq, kk, vv))]


def bwd_autograd(orc):
    for (B, H, S, D, bq, bk, p, seed, dt, scale) in BWD_CASES:
        q, k, v, do, mask = _bwd_case(B, H, S, D, bq, bk, p, seed, dt)
        got = orc.bwd(q, k, v, do, mask, bq, bk, scale)
        want = _autograd_grads(q, k, v, do, mask, bq, bk, scale)
        for name, a, b in zip(("dq", "dk", "dv"), got, want):
            _close(a, b, 1e-11, "%s %s" % (name, dt))


def bwd_finite_diff(orc):
    B, H, S, D, bq, bk, scale = 1, 1, 8, 3, 2, 4, 0.7
    q, k, v, do, mask = _bwd_case(B, H, S, D, bq, bk, 0.7, 41, torch.float64)
    mask[0, 0, 2, :] = 0  # one query block sees nothing
    mask[0, 0, 0, 0] = 1
    dq, dk, dv = orc.bwd(q, k, v, do, mask, bq, bk, scale)
    arrs = {"q": q.numpy().copy(), "k": k.numpy().copy(), "v": v.numpy().copy()}
    grads = {"q": dq, "k": dk, "v": dv}
    g = np.random.default_rng(41)

    def loss():
        out, _ = orc.fwd(arrs["q"], arrs["k"], arrs["v"], mask, bq, bk, scale)
        return float(np.sum(out * do.numpy()))

    h = 1e-5
    for name in ("q", "k", "v"):
        for _ in range(8):
            idx = (0, 0, int(g.integers(S)), int(g.integers(D)))
            x0 = arrs[name][idx]
            arrs[name][idx] = x0 + h
            lp = loss()
            arrs[name][idx] = x0 - h
            lm = loss()
            arrs[name][idx] = x0
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grads[name][idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, grads[name][idx])


def bwd_sums(orc):
    for (B, H, S, D, bq, bk, p, seed, dt, scale) in BWD_CASES:
        q, k, v, do, mask = _bwd_case(B, H, S, D, bq, bk, p, seed, dt)
        mask[0, 0, :, 0] = 0  # key block 0 of head (0, 0): seen by no row
        dq, dk, dv = orc.bwd(q, k, v, do, mask, bq, bk, scale)
        full = expand_mask(mask, bq, bk)
        seen_row = full.any(axis=-1)   # [B,H,S] rows that see a key
        seen_key = full.any(axis=-2)   # [B,H,S] keys some row sees
        _close(dk.sum(axis=2), np.zeros((B, H, D)), 1e-11, "sum dk")
        want_dv = (do.to(torch.float64).numpy() * seen_row[..., None]).sum(axis=2)
        _close(dv.sum(axis=2), want_dv, 1e-11, "sum dv")
        assert np.all(dq[~seen_row] == 0.0)
        assert np.all(dk[~seen_key] == 0.0) and np.all(dv[~seen_key] == 0.0)
        assert (~seen_key).any() and (~seen_row).any()


def bwd_constant_v(orc):
    B, H, S, D, bq, bk, p, seed, dt, scale = BWD_CASES[1]
    q, k, _, do, mask = _bwd_case(B, H, S, D, bq, bk, p, seed, dt)
    v = torch.full((B, H, S, D), -1.75, dtype=torch.float64)
    dq, dk, dv = orc.bwd(q, k, v, do, mask, bq, bk, scale)
    _close(dq, np.zeros_like(dq), 1e-12, "dq")
    _close(dk, np.zeros_like(dk), 1e-12, "dk")
    assert np.abs(dv).max() > 0.1


def bwd_linear_dout(orc):
    B, H, S, D, bq, bk, p, seed, dt, scale = BWD_CASES[0]
    q, k, v, do1, mask = _bwd_case(B, H, S, D, bq, bk, p, seed, dt)
    do2 = _rand((B, H, S, D), 77)
    a, b = 0.75, -2.5
    g1 = orc.bwd(q, k, v, do1, mask, bq, bk, scale)
    g2 = orc.bwd(q, k, v, do2, mask, bq, bk, scale)
    g3 = orc.bwd(q, k, v, a * do1 + b * do2, mask, bq, bk, scale)
    for x1, x2, x3 in zip(g1, g2, g3):
        _close(x3, a * x1 + b * x2, 1e-11, "linearity")


def bwd_sample_match(orc):
    B, H, S, D, bq, bk, p, seed, dt, scale = BWD_CASES[2]
    q, k, v, do, mask = _bwd_case(B, H, S, D, bq, bk, p, seed, dt)
    dq, dk, dv = orc.bwd(q, k, v, do, mask, bq, bk, scale)
    qr = [0, 5, 17, S + 3, 2 * S - 1]
    kr = [1, 16, 31, S, 2 * S - 2]
    sq, sk, sv = orc.bwd_sample(q, k, v, do, mask, bq, bk, scale, qr, kr)
    _close(sq, dq.reshape(-1, D)[qr], 0.0, "dq rows")
    _close(sk, dk.reshape(-1, D)[kr], 0.0, "dk rows")
    _close(sv, dv.reshape(-1, D)[kr], 0.0, "dv rows")


def _autograd_grads_full(q, k, v, do, full, scale):
    """_autograd_grads for an element mask full [B,H,S,S] (True = kept)."""
    full = torch.as_tensor(full)
    qq, kk, vv = (t.to(torch.float64).clone().requires_grad_(True) for t in (q, k, v))
    s = float(np.float32(scale)) * torch.matmul(qq, kk.transpose(-1, -2))
    anyk = full.any(dim=-1, keepdim=True)
    s = s.masked_fill(~full, float("-inf")).masked_fill(~anyk, 0.0)
    pr = torch.softmax(s, dim=-1) * anyk
    out = torch.matmul(pr, vv)
    loss = (out * do.to(torch.float64)).sum()
    return [g.numpy() for g in torch.autograd.grad(loss, (qq, kk, vv))]


def bwd_elem_autograd(orc):
    """Element-mask backward against fp64 autograd through the literal element mask
    (partial tiles, empty blocks, rows that keep nothing, three dtypes)."""
    for (B, H, S, D, bq, bk, nt, seed, dt, scale) in ELEM_CASES:
        q = _rand((B, H, S, D), seed, dt)
        k = _rand((B, H, S, D), seed + 100, dt)
        v = _rand((B, H, S, D), seed + 200, dt)
        do = _rand((B, H, S, D), seed + 300, dt)
        st, pidx, pbits = _elem_case(B, H, S, bq, bk, nt, seed)
        full = expand_elem(st, pidx, pbits, bq, bk)
        got = orc.bwd_elem(q, k, v, do, st, pidx, pbits, bq, bk, scale)
        want = _autograd_grads_full(q, k, v, do, full, scale)
        for name, a, b in zip(("dq", "dk", "dv"), got, want):
            _close(a, b, 1e-11, "elem %s %s" % (name, dt))
        assert (~full.any(axis=-1)).any() or dt != torch.float64  # some row keeps nothing


def _bwd_elem_vs_block(orc, fill):
    B, H, S, D, bq, bk = 1, 2, 64, 8, 16, 32
    q, k, v, do = (_rand((B, H, S, D), s) for s in (81, 82, 83, 84))
    st, pidx, pbits = _elem_case(B, H, S, bq, bk, 2, 85)
    pbits[:] = np.uint32(0xFFFFFFFF) if fill else np.uint32(0)
    got = orc.bwd_elem(q, k, v, do, st, pidx, pbits, bq, bk, 0.5)
    blk = (st != 0) if fill else (st == 1)
    want = orc.bwd(q, k, v, do, blk.astype(np.uint8), bq, bk, 0.5)
    for name, a, b in zip(("dq", "dk", "dv"), got, want):
        _close(a, b, 0.0, "elem vs block %s" % name)


def bwd_elem_tiles_all_set(orc):
    _bwd_elem_vs_block(orc, True)


def bwd_elem_tiles_all_clear(orc):
    _bwd_elem_vs_block(orc, False)


def bwd_elem_token_causal(orc):
    """Exact token-causal (full blocks below the diagonal, one lower-triangular
    tile on it) against the gradients of torch's causal SDPA in fp64."""
    B, H, S, D, b = 1, 2, 96, 8, 32
    q, k, v, do = (_rand((B, H, S, D), s) for s in (91, 92, 93, 94))
    n = S // b
    st = np.broadcast_to(np.tril(np.ones((n, n), dtype=np.uint8)) + np.eye(n, dtype=np.uint8), (B, H, n, n)).copy()
    pidx = np.zeros((B, H, n, n), dtype=np.int32)
    tri = np.tril(np.ones((b, b), dtype=bool))
    pbits = np.packbits(tri, axis=-1, bitorder="little").view(np.uint32).reshape(1, b, b // 32)
    got = orc.bwd_elem(q, k, v, do, st, pidx, pbits, b, b, 0.3)
    qq, kk, vv = (t.clone().requires_grad_(True) for t in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True, scale=float(np.float32(0.3)))
    want = torch.autograd.grad((out * do).sum(), (qq, kk, vv))
    for name, a, w in zip(("dq", "dk", "dv"), got, want):
        _close(a, w.numpy(), 1e-11, "token causal %s" % name)


def bwd_elem_sample_match(orc):
    (B, H, S, D, bq, bk, nt, seed, dt, scale) = ELEM_CASES[1]
    q = _rand((B, H, S, D), seed, dt)
    k = _rand((B, H, S, D), seed + 100, dt)
    v = _rand((B, H, S, D), seed + 200, dt)
    do = _rand((B, H, S, D), seed + 300, dt)
    st, pidx, pbits = _elem_case(B, H, S, bq, bk, nt, seed)
    dq, dk, dv = orc.bwd_elem(q, k, v, do, st, pidx, pbits, bq, bk, scale)
    qr = [0, 7, 33, S + 5, 2 * S - 1]
    kr = [1, 31, 64, S + 2, 2 * S - 3]
    sq, sk, sv = orc.bwd_sample_elem(q, k, v, do, st, pidx, pbits, bq, bk, scale, qr, kr)
    _close(sq, dq.reshape(-1, D)[qr], 0.0, "dq rows")
    _close(sk, dk.reshape(-1, D)[kr], 0.0, "dk rows")
    _close(sv, dv.reshape(-1, D)[kr], 0.0, "dv rows")


ALL = [hand_example, brute_force, sdpa_dense, sdpa_block_causal, block_diagonal, probs_sum,
       constant_v, zero_query, empty_rows, linearity, key_permutation, shift, rows_match_full,
       bf16_widening, fp8_widening, compact_brute, elem_brute, elem_tiles_all_set, elem_tiles_all_clear,
       elem_token_causal, elem_empty_row, elem_rows_match, ragged_hand, ragged_sizes, ragged_one_group,
       ragged_permute, ragged_linear, ragged_tail, ragged_bf16, bwd_autograd, bwd_finite_diff,
       bwd_sums, bwd_constant_v, bwd_linear_dout, bwd_sample_match, bwd_elem_autograd,
       bwd_elem_tiles_all_set, bwd_elem_tiles_all_clear, bwd_elem_token_causal, bwd_elem_sample_match]


def run_all(orc):
    """Run every check; return the names of those that failed (any exception)."""
    failed = []
    for fn in ALL:
        try:
            fn(orc)
        except Exception:  # noqa: BLE001 -- a crash or wrong value both count
            failed.append(fn.__name__)
    return failed


if __name__ == "__main__":  # used by the mutant runner: python oracle_checks.py <lib.so>
    import ctypes
    import sys
    sys.path.insert(0, os.path.dirname(HERE))
    import oracle
    oracle._lib = oracle.configure(ctypes.CDLL(sys.argv[1]))
    print(json.dumps(run_all(oracle)))
