"""Seeded synthetic inputs for block-sparse flash attention.

This module only draws inputs: it holds none of the attention arithmetic, so both
the HIP path (tests, bench) and the CPU oracle can take their inputs from it
without sharing any of the method's code.

Workloads (the pages name no dataset or public benchmark; these synthetic shapes
stand in for the 128-token-chunk, long-sequence setting of "Writing Pallas Kernels
for JAX", section "Designing the Block Specification"):

  tiny_f32       B=1  H=2  S=256    D=64   64x64 blocks   fp32, Bernoulli(0.5) blocks, diagonal on
  dense_bf16     B=4  H=16 S=2048   D=128  128x128 blocks all-ones mask (non-causal)
  causal_bf16    B=2  H=32 S=8192   D=128  128x128 blocks lower-triangular block mask, all heads
  sparse_bf16    B=1  H=16 S=16384  D=128  128x128 blocks window of 4 ending at the diagonal
                                                           + key blocks 0,1 + Bernoulli(0.05)
  long_bf16      B=1  H=8  S=65536  D=64   128x128 blocks (window of 8 ending at the diagonal
                                                           + every 16th key block + Bernoulli(0.01))
                                                           restricted to kj <= qi

Element-level mask workload (block states + bit tiles, see bsattn.h):

  causal_elem_bf16  B=2 H=32 S=8192 D=128 128x128 blocks  exact token-causal: blocks
                    below the diagonal full, diagonal blocks partial through one shared
                    lower-triangular tile (query i keeps keys j <= i)

Ragged dot workload (grouped matrix multiplication):

  ragged_bf16       M=32768 K=2048 N=2048 G=8 bf16; rows routed to expert g with
                    probability ~ 1/(g+1) (seed 3)

Recipe: Q, K, V ~ N(0, 1) drawn in that order from one torch CPU generator seeded 0,
each of shape [B,H,S,D] in fp32, then rounded to bf16 (round-to-nearest-even) for
the bf16 workloads.  Random mask extras come from a separate torch CPU generator
(seed 0 for tiny_f32, 7 for sparse_bf16, 11 for long_bf16): one uniform draw of
shape [B,H,n_q,n_k], a block active where u < p.  scale = 1/sqrt(D) as fp32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    D: int
    block_q: int
    block_k: int
    dtype: str  # "f32" or "bf16"
    mask_kind: str
    mask_seed: int = 0

    @property
    def n_q(self) -> int:
        return self.S // self.block_q

    @property
    def n_k(self) -> int:
        return self.S // self.block_k

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.D)))

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 2, 256, 64, 64, 64, "f32", "bernoulli_diag", 0),
    "dense_bf16": Workload("dense_bf16", 4, 16, 2048, 128, 128, 128, "bf16", "ones"),
    "causal_bf16": Workload("causal_bf16", 2, 32, 8192, 128, 128, 128, "bf16", "causal"),
    "sparse_bf16": Workload("sparse_bf16", 1, 16, 16384, 128, 128, 128, "bf16",
                            "window_global_random", 7),
    "long_bf16": Workload("long_bf16", 1, 8, 65536, 64, 128, 128, "bf16",
                          "causal_window_strided_random", 11),
}

ORDER = ["tiny_f32", "dense_bf16", "causal_bf16", "sparse_bf16", "long_bf16"]

ELEM_WORKLOADS = {
    "causal_elem_bf16": Workload("causal_elem_bf16", 2, 32, 8192, 128, 128, 128, "bf16",
                                 "token_causal"),
}


def make_qkv(B, H, S, D, dtype=torch.bfloat16, seed=0):
    """Q, K, V ~ N(0,1) [B,H,S,D], drawn in that order from one CPU generator."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, S, D, generator=g)
    k = torch.randn(B, H, S, D, generator=g)
    v = torch.randn(B, H, S, D, generator=g)
    if dtype != torch.float32:
        q, k, v = q.to(dtype), k.to(dtype), v.to(dtype)
    return q, k, v


def _uniform(B, H, n_q, n_k, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.rand(B, H, n_q, n_k, generator=g)


def _grid(n_q, n_k):
    i = torch.arange(n_q).view(n_q, 1)
    j = torch.arange(n_k).view(1, n_k)
    return i, j


def mask_bernoulli(B, H, n_q, n_k, p, seed, diag=False):
    m = _uniform(B, H, n_q, n_k, seed) < p
    if diag:
        i, j = _grid(n_q, n_k)
        m = m | (i == j)
    return m.to(torch.uint8)


def mask_ones(B, H, n_q, n_k):
    return torch.ones(B, H, n_q, n_k, dtype=torch.uint8)


def mask_causal(B, H, n_q, n_k):
    i, j = _grid(n_q, n_k)
    return (j <= i).to(torch.uint8).expand(B, H, n_q, n_k).contiguous()


def mask_window_global_random(B, H, n_q, n_k, window=4, n_global=2, p=0.05, seed=7):
    i, j = _grid(n_q, n_k)
    band = (j <= i) & (j >= i - (window - 1))
    glob = j < n_global
    extra = _uniform(B, H, n_q, n_k, seed) < p
    return (band | glob | extra).to(torch.uint8)


def mask_causal_window_strided_random(B, H, n_q, n_k, window=8, stride=16, p=0.01, seed=11):
    i, j = _grid(n_q, n_k)
    band = (j <= i) & (j >= i - (window - 1))
    strided = (j % stride) == 0
    extra = _uniform(B, H, n_q, n_k, seed) < p
    return ((band | strided | extra) & (j <= i)).to(torch.uint8)


def make_mask(w: Workload):
    B, H, n_q, n_k = w.B, w.H, w.n_q, w.n_k
    if w.mask_kind == "bernoulli_diag":
        return mask_bernoulli(B, H, n_q, n_k, 0.5, w.mask_seed, diag=True)
    if w.mask_kind == "ones":
        return mask_ones(B, H, n_q, n_k)
    if w.mask_kind == "causal":
        return mask_causal(B, H, n_q, n_k)
    if w.mask_kind == "window_global_random":
        return mask_window_global_random(B, H, n_q, n_k, seed=w.mask_seed)
    if w.mask_kind == "causal_window_strided_random":
        return mask_causal_window_strided_random(B, H, n_q, n_k, seed=w.mask_seed)
    if w.mask_kind == "token_causal":  # the non-empty blocks of the element mask
        return mask_causal(B, H, n_q, n_k)
    raise ValueError(w.mask_kind)


@dataclass(frozen=True)
class RaggedWorkload:
    name: str
    M: int
    K: int
    N: int
    G: int
    seed: int = 0


# Ragged dot ("Pallas-Triton kernels and kernel auto-tuning", section "Ragged Dot"):
# a mixture-of-experts layer's shape: M tokens routed to G experts.
RAGGED_WORKLOADS = {
    "ragged_bf16": RaggedWorkload("ragged_bf16", 32768, 2048, 2048, 8, 3),
}


def make_ragged(w: RaggedWorkload):
    """lhs [M, K], rhs [G, K, N] ~ N(0, 1) rounded to bf16 (one CPU generator,
    seed w.seed, lhs first), and group sizes: each of the M rows goes to expert g
    with probability proportional to 1 / (g + 1) (a skewed routing, seeded),
    counted per expert (int32 [G], sum M)."""
    g = torch.Generator().manual_seed(w.seed)
    lhs = torch.randn(w.M, w.K, generator=g).to(torch.bfloat16)
    rhs = torch.randn(w.G, w.K, w.N, generator=g).to(torch.bfloat16)
    probs = 1.0 / torch.arange(1, w.G + 1, dtype=torch.float64)
    choice = torch.multinomial(probs / probs.sum(), w.M, replacement=True, generator=g)
    sizes = torch.bincount(choice, minlength=w.G).to(torch.int32)
    return lhs, rhs, sizes


def pack_tiles(bits):
    """Bool tiles [n, block_q, block_k] -> int32 words [n, block_q, block_k / 32],
    bit c % 32 of word c / 32 = element c (little-endian bit order)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=bool))
    n, bq, bk = b.shape
    words = np.packbits(b, axis=-1, bitorder="little").view(np.uint32).reshape(n, bq, bk // 32)
    return torch.from_numpy(words.view(np.int32).copy())


def make_elem_mask(w: Workload):
    """(block_states uint8, partial_index int32, partial_bits int32) of an
    element-level workload."""
    B, H, n_q, n_k = w.B, w.H, w.n_q, w.n_k
    if w.mask_kind == "token_causal":
        assert w.block_q == w.block_k
        i, j = _grid(n_q, n_k)
        states = ((j < i).to(torch.uint8) + 2 * (j == i).to(torch.uint8)).expand(B, H, n_q, n_k)
        tri = np.tril(np.ones((w.block_q, w.block_k), dtype=bool))[None]
        return (states.contiguous(), torch.zeros(B, H, n_q, n_k, dtype=torch.int32),
                pack_tiles(tri))
    raise ValueError(w.mask_kind)


def kept_elements(states, partial_index, partial_bits, block_q, block_k) -> int:
    """Number of kept (query, key) elements of an element-level mask."""
    st = torch.as_tensor(states).to(torch.int64)
    full = int((st == 1).sum().item()) * block_q * block_k
    words = np.asarray(torch.as_tensor(partial_bits).numpy()).view(np.uint32)
    per_tile = np.unpackbits(words.view(np.uint8).reshape(words.shape[0], -1), axis=-1).sum(-1)
    pidx = torch.as_tensor(partial_index)[st > 1].numpy()
    pidx = np.clip(pidx, 0, words.shape[0] - 1)
    return full + int(per_tile[pidx].sum())


def make_inputs(w: Workload, seed=0):
    q, k, v = make_qkv(w.B, w.H, w.S, w.D, w.torch_dtype, seed)
    return q, k, v, make_mask(w)


def active_elements(mask, block_q, block_k) -> int:
    """Number of active (query, key) score elements: active blocks x block area."""
    return int(torch.as_tensor(mask).ne(0).sum().item()) * block_q * block_k


def flops(mask, block_q, block_k, D) -> int:
    """Algorithmic FLOPs: 4*D per active score element (2*D for Q.K, 2*D for P.V)."""
    return 4 * D * active_elements(mask, block_q, block_k)


def sample_rows(B, H, S, block_q, n, seed=1234, mask=None):
    """A seeded sample of flat query rows (b*H + h)*S + s for full-size checks:
    the first and last rows, rows on query-tile edges, rows of the mask row with
    the most active blocks, and random rows."""
    g = np.random.default_rng(seed)
    total = B * H * S
    picks = {0, total - 1, S - 1, min(S, total - 1)}
    if mask is not None:
        cnt = torch.as_tensor(mask).ne(0).sum(-1).reshape(-1).numpy()  # per (b,h,qi)
        n_q = S // block_q
        for r in np.argsort(-cnt, kind="stable")[:4]:
            bh, qi = divmod(int(r), n_q)
            picks.add(bh * S + qi * block_q)
            picks.add(bh * S + qi * block_q + block_q - 1)
    while len(picks) < n:
        bh = int(g.integers(0, B * H))
        s = int(g.integers(0, S))
        picks.add(bh * S + s)
        if len(picks) < n:  # a query-tile edge row too
            picks.add(bh * S + (s // block_q) * block_q + (block_q - 1 if s % 2 else 0))
    return np.array(sorted(picks), dtype=np.int64)
