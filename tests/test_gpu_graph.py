"""Calls recorded into a HIP graph (torch.cuda.CUDAGraph) and replayed: every
replay must give, bit for bit, what the same call gives eagerly (the float
atomics of the bias-table gradients aside, which are compared to tolerance).

Between replays the test zeroes the graph's outputs (so a replay that skips
work is seen), runs eager calls of other sizes and kinds on the default
stream (which move the eager counter rotation on and reuse its scratch), and
synchronises.  A captured call has a scratch area of its own whose queue
counters its first recorded kernel clears, so none of that may change a
replay's result.
"""
import numpy as np
import pytest

import workloads
from helpers import device_case, log, to_torch

torch = pytest.importorskip("torch")
hstu = pytest.importorskip("generative_recommendation_attention_amd")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

REPLAYS = 4


def bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def capture(fn):
    """Warm fn up eagerly on a side stream, then record it; returns the graph
    and the tensors fn returned during capture (the graph's outputs)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    torch.cuda.synchronize()
    return g, outs


def eager_noise(i):
    """Eager calls of other sizes between replays (small: one-kernel form;
    300 sequences: the work-list kernel; a backward: two counter sets)."""
    lengths = [50 + 17 * i, 3, 200] if i % 2 == 0 else \
        list(np.random.default_rng(i).integers(1, 60, size=300))
    c = workloads.make_case(lengths, 2, 64, "bf16", seed=3000 + i)
    q, k, v, off = device_case(c)
    hstu.hstu_attn_fwd(q, k, v, off, c.alpha, c.n)
    hstu.hstu_attn_bwd(q, k, v, q, off, c.alpha, c.n)


def check_replays(fn, exact=None, close=None, name=""):
    """exact / close: indices of the outputs compared bit for bit / to within
    1e-3 of their largest magnitude (float-atomic sums, whose order varies)."""
    ref = [t.clone() for t in fn()]
    torch.cuda.synchronize()
    g, outs = capture(fn)
    exact = range(len(outs)) if exact is None else exact
    close = close or []
    for i in range(REPLAYS):
        for o in outs:
            o.zero_()
        eager_noise(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j in exact:
            assert torch.equal(bits(outs[j]), bits(ref[j])), f"{name}: replay {i}, output {j}"
        for j in close:
            err = (outs[j] - ref[j]).abs().max().item()
            assert err <= 1e-3 * max(ref[j].abs().max().item(), 1e-30), \
                f"{name}: replay {i}, output {j}: {err}"
    log(f"{name}: {REPLAYS} replays match the eager call")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("size", ["small", "many"])
def test_forward_replays(dtype, size):
    lengths = [100, 37, 300] if size == "small" else \
        list(np.random.default_rng(5).integers(0, 90, size=300))
    c = workloads.make_case(lengths, 2, 64 if dtype != "fp16" else 128, dtype, seed=3100,
                            sigma=0.5 if dtype == "fp16" else 1.0)
    q, k, v, off = device_case(c)
    check_replays(lambda: [hstu.hstu_attn_fwd(q, k, v, off, c.alpha, c.n)],
                  name=f"forward {dtype} {size}")


def test_masked_and_biased_forms_replay():
    c = workloads.make_case([300, 129, 64, 1], 2, 64, "bf16", seed=3110)
    q, k, v, off = device_case(c)
    tg = torch.tensor([64, 128, 0, 1], dtype=torch.int32, device="cuda")
    r = workloads.make_rab_inputs(c.offsets, 200, 12, seed=3111)
    ts = torch.from_numpy(r.timestamps).cuda()
    wp = torch.from_numpy(r.pos_bias).cuda()
    wt = torch.from_numpy(r.time_bias).cuda()
    check_replays(lambda: [hstu.hstu_attn_fwd_targets(q, k, v, off, tg, c.alpha, c.n),
                           hstu.hstu_attn_fwd_rab(q, k, v, off, ts, wp, wt, c.alpha, c.n),
                           hstu.hstu_attn_fwd_rab_targets(q, k, v, off, tg, ts, wp, wt, c.alpha,
                                                          c.n)],
                  name="targets, bias, bias + targets")


def test_cached_and_dense_replay():
    cc = workloads.make_cached_case([50, 0, 130], [20, 7, 64], 2, 64, "bf16", seed=3120, n=200.0)
    cand = cc.cand
    cq, ck, cv = (to_torch(x, "bf16") for x in (cand.q, cand.k, cand.v))
    coff = torch.from_numpy(cand.offsets).cuda()
    kc, vc = to_torch(cc.k_cache, "bf16"), to_torch(cc.v_cache, "bf16")
    hoff = torch.from_numpy(cc.hist_offsets).cuda()
    r, hist_ts = workloads.make_cached_rab_inputs(cc.hist_offsets, cand.offsets, 150, 10,
                                                  seed=3122)
    ts, hts = torch.from_numpy(r.timestamps).cuda(), torch.from_numpy(hist_ts).cuda()
    wp, wt = torch.from_numpy(r.pos_bias).cuda(), torch.from_numpy(r.time_bias).cuda()
    dc = workloads.make_case([256] * 3, 2, 64, "bf16", seed=3121)
    dq, dk, dv, _ = device_case(dc)
    qd, kd, vd = (x.reshape(3, 256, 2, 64).permute(0, 2, 1, 3).contiguous() for x in (dq, dk, dv))
    check_replays(lambda: [hstu.hstu_attn_fwd_cached(cq, ck, cv, coff, kc, vc, hoff, cand.alpha,
                                                     cand.n),
                           hstu.hstu_attn_fwd_rab_cached(cq, ck, cv, coff, kc, vc, hoff, ts, hts,
                                                         wp, wt, cand.alpha, cand.n),
                           hstu.hstu_attn_fwd_dense(qd, kd, vd, dc.alpha, dc.n)],
                  name="cached history, cached history with bias, dense")


@pytest.mark.parametrize("size", ["small", "many"])
def test_backward_replays(size):
    lengths = [300, 37, 129] if size == "small" else \
        list(np.random.default_rng(6).integers(0, 90, size=300))
    c = workloads.make_case(lengths, 2, 64, "bf16", seed=3130)
    q, k, v, off = device_case(c)
    dout = to_torch(workloads.make_case(lengths, 2, 64, "bf16", seed=3131).q, "bf16")
    check_replays(lambda: list(hstu.hstu_attn_bwd(q, k, v, dout, off, c.alpha, c.n)),
                  name=f"backward {size}")


def test_forward_then_backward_with_bias_in_one_graph():
    c = workloads.make_case([400, 77, 1, 250], 2, 64, "bf16", seed=3140)
    q, k, v, off = device_case(c)
    dout = to_torch(workloads.make_case(list(c.lengths), 2, 64, "bf16", seed=3141).q, "bf16")
    r = workloads.make_rab_inputs(c.offsets, 300, 16, seed=3142)
    ts = torch.from_numpy(r.timestamps).cuda()
    wp = torch.from_numpy(r.pos_bias).cuda()
    wt = torch.from_numpy(r.time_bias).cuda()

    def fn():
        out = hstu.hstu_attn_fwd_rab(q, k, v, off, ts, wp, wt, c.alpha, c.n)
        return [out] + list(hstu.hstu_attn_bwd_rab(q, k, v, dout, off, ts, wp, wt, c.alpha,
                                                   c.n))
    check_replays(fn, exact=[0, 1, 2, 3], close=[4, 5], name="bias forward + backward")


def test_layer_in_one_graph():
    """Input projection, attention on its q, k, v, output projection: one
    recorded layer, replayed against the eager layer."""
    T_lengths = [300, 77, 129]
    H, d, dm = 4, 64, 256
    c = workloads.make_case(T_lengths, H, d, "bf16", seed=3150)
    off = torch.from_numpy(c.offsets).cuda()
    T = c.total
    g = torch.Generator(device="cpu").manual_seed(3151)
    x = (torch.randn(T, dm, generator=g) * 0.5).to(torch.bfloat16).cuda()
    w1 = (torch.randn(4 * H * d, dm, generator=g) / 16).to(torch.bfloat16).cuda()
    b1 = (torch.randn(4 * H * d, generator=g) * 0.1).cuda()
    w2 = (torch.randn(dm, H * d, generator=g) / 16).to(torch.bfloat16).cuda()
    b2 = (torch.randn(dm, generator=g) * 0.1).cuda()
    gamma = (1.0 + 0.1 * torch.randn(H * d, generator=g)).cuda()
    beta = (0.1 * torch.randn(H * d, generator=g)).cuda()

    def fn():
        u, v, q, k = hstu.hstu_layer_in_proj(x, w1, b1, H, d)
        a = hstu.hstu_attn_fwd(q, k, v, off, c.alpha, c.n)
        return [hstu.hstu_layer_out_proj(a, u, x, gamma, beta, 1e-5, w2, b2)]
    check_replays(fn, name="layer")
