"""The four bf16 block-mask workloads at full size, every output element against
the fp64 oracle: dense (B4 H16 S2048 D128), block-causal (B2 H32 S8192 D128),
block-sparse (B1 H16 S16384 D128) and long-context sparse (B1 H8 S65536 D64).

For each workload the oracle computes the whole output once (a module-scoped
cache; block-causal is about a minute on the host's cores), then the GPU runs
the tile config the autotuner picks for that workload (the launch bench.py
times) and every other row-pair config legal for it.  Max and mean |error| are
taken over all B*H*S*D output elements, the lse error over all rows, against
the bf16 tolerances (out max 1e-2, mean 1e-3, lse 1e-3)."""
import time

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import bs, compare, ensure_built, say

pytestmark = pytest.mark.gpu

_REF = {}


def _reference(name):
    """Inputs (host) and the oracle's full output of workload `name`."""
    if name not in _REF:
        _REF.clear()  # one workload's fp64 output at a time (block-causal: 0.5 GiB)
        w = W.WORKLOADS[name]
        q, k, v, mask = W.make_inputs(w)
        say("oracle", name, "full output on", oracle.max_threads(), "threads ...")
        t0 = time.perf_counter()
        ro, rl = oracle.fwd(q, k, v, mask, w.block_q, w.block_k, w.scale)
        say("oracle", name, "done in %.1f s" % (time.perf_counter() - t0))
        _REF[name] = (w, q, k, v, mask, ro, rl)
    return _REF[name]


@pytest.mark.parametrize("name", ["dense_bf16", "causal_bf16", "sparse_bf16", "long_bf16"])
def test_full_output_tuned_and_pair_configs(name):
    ensure_built()
    w, q, k, v, mask, ro, rl = _reference(name)
    qd, kd, vd, md = q.cuda(), k.cuda(), v.cuda(), mask.cuda()
    say("autotune", name)
    best, rows = bs.autotune(qd, kd, vd, md, w.block_q, w.block_k, w.scale, warmup=1, iters=3)
    cfgs = [best.as_tuple()]
    cfgs += [c.as_tuple() for c in bs.list_configs(torch.bfloat16, w.D, w.block_q, w.block_k)
             if c.tile_q == 256 and c.as_tuple() != best.as_tuple()]
    for cfg in cfgs:
        say("full output", name, cfg, "(tuned)" if cfg == cfgs[0] else "")
        out, lse = bs.fwd(qd, kd, vd, md, w.block_q, w.block_k, w.scale, config=cfg)
        torch.cuda.synchronize()
        stats = compare(out, lse, ro, rl, "bf16", "%s %s" % (name, cfg))
        say("  ", stats)
        del out, lse
    bs.clear_tune_cache()


def test_full_output_token_causal_element_mask():
    """The exact token-causal element-mask workload (B2 H32 S8192 D128, 128x128 blocks:
    full blocks below the diagonal, one shared lower-triangular bit tile on it) at full
    size: every output element of every row-pair element config (bench.py times these
    and keeps the fastest) and of the first four-wave one against the oracle's
    element-mask forward; the call with no config (the built-in default) equals the
    (256, 64, 8, 2) row pair bit for bit."""
    ensure_built()
    _REF.clear()
    w = W.ELEM_WORKLOADS["causal_elem_bf16"]
    q, k, v, _ = W.make_inputs(w)
    st, pidx, pbits = W.make_elem_mask(w)
    say("oracle", w.name, "full output on", oracle.max_threads(), "threads ...")
    t0 = time.perf_counter()
    ro, rl = oracle.fwd_elem(q, k, v, st, pidx, pbits, w.block_q, w.block_k, w.scale)
    say("oracle", w.name, "done in %.1f s" % (time.perf_counter() - t0))
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    sd, pd, bd = st.cuda(), pidx.cuda(), pbits.cuda()
    listed = [c.as_tuple() for c in bs.list_configs_elem(torch.bfloat16, w.D, w.block_q, w.block_k)]
    cfgs = [c for c in listed if c[0] == 256] + [c for c in listed if c[0] != 256][:1]
    assert len(cfgs) >= 3
    outs = {}
    for cfg in cfgs:
        say("full output", w.name, cfg)
        out, lse = bs.fwd_elem(qd, kd, vd, sd, pd, bd, w.block_q, w.block_k, w.scale, config=cfg)
        torch.cuda.synchronize()
        stats = compare(out, lse, ro, rl, "bf16", "%s %s" % (w.name, cfg))
        say("  ", stats)
        if cfg == (256, 64, 8, 2):
            outs[cfg] = (out, lse)
        else:
            del out, lse
    # no config: the built-in default, the row pair with 64-key steps
    out, lse = bs.fwd_elem(qd, kd, vd, sd, pd, bd, w.block_q, w.block_k, w.scale)
    torch.cuda.synchronize()
    ref_out, ref_lse = outs[(256, 64, 8, 2)]
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
