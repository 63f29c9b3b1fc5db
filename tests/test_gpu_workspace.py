"""The library's scratch areas: growth, release, streams and allocation
failure.  Every result is compared bit for bit with the same call made on a
settled area, since none of these may change what a call computes."""
import os

import numpy as np
import pytest

import workloads
from helpers import device_case

torch = pytest.importorskip("torch")
hstu = pytest.importorskip("generative_recommendation_attention_amd")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


def bits(t):
    return t.view(torch.int16)


def cases():
    small = workloads.make_case([100, 37, 300], 2, 64, "bf16", seed=4000)
    big = workloads.make_case(list(np.random.default_rng(40).integers(1, 120, size=600)), 2, 64,
                              "bf16", seed=4001)
    return small, big


def fwd(case, stream=None):
    q, k, v, off = device_case(case)
    return hstu.hstu_attn_fwd(q, k, v, off, case.alpha, case.n, stream=stream)


def test_growth_and_release_keep_results():
    """Small call, a call with more sequences (the area grows), the small
    one again, a release, then both again: identical outputs throughout."""
    small, big = cases()
    ref_s = fwd(small).clone()
    ref_b = fwd(big).clone()
    torch.cuda.synchronize()
    for _ in range(2):
        assert torch.equal(bits(fwd(small)), bits(ref_s))
        assert torch.equal(bits(fwd(big)), bits(ref_b))
        torch.cuda.synchronize()
        hstu.hstu_release_workspace()
    q, k, v, off = device_case(small)
    dout = q.clone()
    g1 = hstu.hstu_attn_bwd(q, k, v, dout, off, small.alpha, small.n)
    torch.cuda.synchronize()
    hstu.hstu_release_workspace()
    g2 = hstu.hstu_attn_bwd(q, k, v, dout, off, small.alpha, small.n)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(bits(a), bits(b))


def test_graph_replays_after_release():
    """A recorded call keeps its own area, so releasing the per-stream areas
    does not touch it."""
    small, big = cases()
    q, k, v, off = device_case(big)
    ref = hstu.hstu_attn_fwd(q, k, v, off, big.alpha, big.n).clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        hstu.hstu_attn_fwd(q, k, v, off, big.alpha, big.n)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = hstu.hstu_attn_fwd(q, k, v, off, big.alpha, big.n)
    torch.cuda.synchronize()
    for _ in range(3):
        hstu.hstu_release_workspace()
        fwd(small)   # a new per-stream area
        torch.cuda.synchronize()
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(ref))


def test_two_streams_at_once():
    """Calls on two streams overlap, each with its own area."""
    small, big = cases()
    ref_s = fwd(small).clone()
    ref_b = fwd(big).clone()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for i in range(4):
        with torch.cuda.stream(s1):
            outs.append(("s", fwd(small, stream=s1)))
        with torch.cuda.stream(s2):
            outs.append(("b", fwd(big, stream=s2)))
    torch.cuda.synchronize()
    for kind, o in outs:
        assert torch.equal(bits(o), bits(ref_s if kind == "s" else ref_b))


def test_allocation_failure_is_reported_and_recoverable():
    """A stream with no area yet cannot get one (allocation made to fail):
    the call raises with the no-memory status and enqueues nothing; the
    same call succeeds once allocation works again."""
    small, _ = cases()
    ref = fwd(small).clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        os.environ["HSTU_FAIL_ALLOC"] = "1"
        try:
            with pytest.raises(hstu.HstuError) as e:
                fwd(small, stream=s)
            assert e.value.status == hstu.HSTU_ERR_NO_MEMORY
        finally:
            del os.environ["HSTU_FAIL_ALLOC"]
        out = fwd(small, stream=s)
    torch.cuda.synchronize()
    assert torch.equal(bits(out), bits(ref))
