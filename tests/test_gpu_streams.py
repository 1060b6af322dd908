"""Calls on caller-created HIP streams (the `stream` argument of every entry point):
several calls in flight at once on two streams, each with its own workspace and
outputs, give bit for bit the results of the same calls run one after another on
the default stream (the boundary promises that calls on different streams may run
concurrently when their workspaces and outputs differ)."""
import numpy as np
import pytest
import torch

from gpu_util import bs, ensure_built, rand_mask, rand_qkv

pytestmark = pytest.mark.gpu


def _case(seed, S=1024, D=128, b=128):
    q, k, v = (t.cuda() for t in rand_qkv(2, 4, S, D, torch.bfloat16, seed))
    mask = rand_mask(2, 4, S // b, S // b, 0.5, seed, empty_rows=[(0, 1, 2)]).cuda()
    return q, k, v, mask


def test_forward_and_backward_on_two_streams():
    ensure_built()
    b = 128
    cases = [_case(s) for s in (201, 202, 203, 204)]
    do = [torch.randn_like(c[0]) for c in cases]
    ref = []
    for (q, k, v, m), g in zip(cases, do):
        out, lse = bs.fwd(q, k, v, m, b, b)
        grads = bs.bwd(q, k, v, out, lse, g, m, b, b)
        ref.append((out, lse) + tuple(grads))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    got = []
    for i, ((q, k, v, m), g) in enumerate(zip(cases, do)):
        s = streams[i % 2]
        out, lse = bs.fwd(q, k, v, m, b, b, stream=s)
        grads = bs.bwd(q, k, v, out, lse, g, m, b, b, stream=s)
        got.append((out, lse) + tuple(grads))
    torch.cuda.synchronize()
    for r, x in zip(ref, got):
        for a, c in zip(r, x):
            assert torch.equal(a, c)


def test_planned_fp8_and_ragged_on_a_side_stream():
    ensure_built()
    b, S = 128, 1024
    q, k, v, m = _case(211, S=S)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    # forward on a plan made on the side stream
    ref_o, ref_l = bs.fwd(q, k, v, m, b, b)
    plan = bs.plan(m, S, b, b, stream=s)
    o, l = bs.fwd_planned(q, k, v, plan, b, b, stream=s)
    # fp8 forward
    q8, k8, v8 = (t.float().to(torch.float8_e4m3fn) for t in (q, k, v))
    torch.cuda.synchronize()
    ref8 = bs.fwd_fp8(q8, k8, v8, m, b, b)
    s.wait_stream(torch.cuda.current_stream())
    got8 = bs.fwd_fp8(q8, k8, v8, m, b, b, stream=s)
    # ragged dot
    g = torch.Generator().manual_seed(212)
    x = torch.randn(700, 256, generator=g).to(torch.bfloat16).cuda()
    w = torch.randn(3, 256, 384, generator=g).to(torch.bfloat16).cuda()
    sizes = torch.tensor([300, 0, 350], dtype=torch.int32).cuda()
    torch.cuda.synchronize()
    ref_r = bs.ragged_dot(x, w, sizes)
    s.wait_stream(torch.cuda.current_stream())
    got_r = bs.ragged_dot(x, w, sizes, stream=s)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
    assert torch.equal(got8[0], ref8[0]) and torch.equal(got8[1], ref8[1])
    assert torch.equal(got_r, ref_r)
    assert torch.all(got_r[650:] == 0) and not np.isnan(got_r.float().cpu().numpy()).any()
