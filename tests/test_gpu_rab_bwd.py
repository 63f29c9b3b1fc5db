"""Parity of the backward with the relative attention bias against the fp64
CPU oracle, through the C ABI: dq, dk, dv element by element, and the two
tables' gradients (HSTU paper translation, Appendix G: the bias is recomputed
in the backward and its gradients accumulated on chip).

The table gradients are float sums taken with atomics, so they are compared
within the tolerance, not bit for bit.  Properties: zero tables give the
plain backward's dq, dk, dv bit for bit; with a position entry for every
distance the two tables' gradients have the same total.
"""
import numpy as np
import pytest

import oracle
import workloads
from helpers import assert_close, device_case, from_torch, log, to_torch

torch = pytest.importorskip("torch")
hstu = pytest.importorskip("generative_recommendation_attention_amd")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

LENGTHS = [1, 37, 300, 129, 0, 200, 64]


def make(lengths, heads, d, dtype, npos, ntime, seed):
    sigma = 0.5 if dtype == "fp16" else 1.0
    case = workloads.make_case(lengths, heads, d, dtype, seed=seed, sigma=sigma)
    dout = workloads.make_case(lengths, heads, d, dtype, seed=seed + 1, sigma=sigma).q
    r = workloads.make_rab_inputs(case.offsets, npos, ntime, seed=seed + 2)
    return case, dout, r


def run_bwd_rab(case, dout, r):
    q, k, v, off = device_case(case)
    do = to_torch(dout, case.dtype)
    ts = torch.from_numpy(r.timestamps).cuda()
    wp = torch.from_numpy(r.pos_bias).cuda()
    wt = torch.from_numpy(r.time_bias).cuda()
    res = hstu.hstu_attn_bwd_rab(q, k, v, do, off, ts, wp, wt, case.alpha, case.n)
    torch.cuda.synchronize()
    return res


def compare(case, dout, r, res, what):
    ref = oracle.bwd_rab(case.q, case.k, case.v, dout, case.offsets, r.timestamps, r.pos_bias,
                         r.time_bias, case.heads, case.d, case.alpha, case.n, case.dtype)
    for name, g, rf in zip(("dq", "dk", "dv"), res[:3], ref[:3]):
        assert_close(from_torch(g, case.dtype), rf, case.dtype, f"{what} {name}")
    for name, g, rf in zip(("d_pos_bias", "d_time_bias"), res[3:], ref[3:]):
        got = g.cpu().numpy().astype(np.float64)
        mr, l2 = assert_close(got, rf, case.dtype, f"{what} {name}")
        log(f"  {name}: max|err|/max|ref| = {mr:.2e}, rel L2 = {l2:.2e}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("npos,ntime", [(400, 16), (50, 32), (1, 1)])
def test_rab_bwd_full_compare(dtype, d, npos, ntime):
    case, dout, r = make(LENGTHS, 2, d, dtype, npos, ntime, seed=1500 + d + npos)
    log(f"rab bwd {dtype} d={d} npos={npos} ntime={ntime}")
    compare(case, dout, r, run_bwd_rab(case, dout, r), f"rab bwd {dtype} d{d}")


def test_rab_bwd_decreasing_timestamps():
    case, dout, r = make([150, 90], 2, 64, "bf16", 200, 12, seed=1510)
    r.timestamps = (5_000_000 - 11 * np.arange(case.total)).astype(np.int32)
    compare(case, dout, r, run_bwd_rab(case, dout, r), "rab bwd decreasing timestamps")


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("fp16", 128), ("fp32", 64)])
def test_rab_bwd_zero_tables_match_plain_bitwise(dtype, d):
    case, dout, r = make(LENGTHS + [513], 3, d, dtype, 30, 5, seed=1520)
    r.pos_bias[:] = 0
    r.time_bias[:] = 0
    got = run_bwd_rab(case, dout, r)
    q, k, v, off = device_case(case)
    plain = hstu.hstu_attn_bwd(q, k, v, to_torch(dout, dtype), off, case.alpha, case.n)
    torch.cuda.synchronize()
    for a, b in zip(got[:3], plain):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_rab_bwd_many_sequences_worklist_path():
    lengths = list(np.random.default_rng(4).integers(0, 150, size=300))
    case, dout, r = make(lengths, 2, 64, "bf16", 160, 12, seed=1530)
    compare(case, dout, r, run_bwd_rab(case, dout, r), "rab bwd 300 sequences")


def test_rab_bwd_long_sequences_tables():
    """Two 2048-token sequences, heads 4: the tables' gradients element by
    element (thousands of distances, every bucket), dq/dk/dv on sampled rows."""
    case, dout, r = make([2048, 1500], 4, 64, "bf16", 2048, 16, seed=1540)
    log("rab bwd 2048 + 1500, heads 4")
    res = run_bwd_rab(case, dout, r)
    ref = oracle.bwd_rab(case.q, case.k, case.v, dout, case.offsets, r.timestamps, r.pos_bias,
                         r.time_bias, 4, 64, case.alpha, case.n, "bf16")
    for name, g, rf in zip(("d_pos_bias", "d_time_bias"), res[3:], ref[3:]):
        mr, l2 = assert_close(g.cpu().numpy().astype(np.float64), rf, "bf16", name)
        log(f"  {name}: max|err|/max|ref| = {mr:.2e}, rel L2 = {l2:.2e}")
    for name, g, rf in zip(("dq", "dk", "dv"), res[:3], ref[:3]):
        assert_close(from_torch(g, "bf16"), rf, "bf16", name)


def test_rab_bwd_workload_full_compare_and_totals():
    """16 x 4096, heads 4, d 64, bf16 (the forward's bias workload): every
    element of dq, dk, dv and of both table gradients against the fp64
    oracle (about 45 s of oracle time on 16 host threads), and equal totals
    of the two table gradients."""
    case, r = workloads.rab_workload()
    dout = workloads.make_case([4096] * 16, 4, 64, "bf16", seed=1550).q
    log("rab bwd workload 16 x 4096 (whole output)")
    res = run_bwd_rab(case, dout, r)
    ref = oracle.bwd_rab(case.q, case.k, case.v, dout, case.offsets, r.timestamps, r.pos_bias,
                         r.time_bias, 4, 64, case.alpha, case.n, "bf16")
    for name, g, rf in zip(("dq", "dk", "dv"), res[:3], ref[:3]):
        mr, l2 = assert_close(from_torch(g, "bf16"), rf, "bf16", f"rab bwd workload {name}")
        log(f"  {name}: max|err|/max|ref| = {mr:.2e}, rel L2 = {l2:.2e}")
    for name, g, rf in zip(("d_pos_bias", "d_time_bias"), res[3:], ref[3:]):
        mr, l2 = assert_close(g.cpu().numpy().astype(np.float64), rf, "bf16",
                              f"rab bwd workload {name}")
        log(f"  {name}: max|err|/max|ref| = {mr:.2e}, rel L2 = {l2:.2e}")
    sp = float(res[3].double().sum())
    st = float(res[4].double().sum())
    scale = float(res[3].double().abs().sum())
    assert abs(sp - st) <= 1e-4 * scale, (sp, st, scale)


def test_rab_bwd_qkv_deterministic():
    case, dout, r = make([1000, 300], 4, 64, "bf16", 500, 16, seed=1560)
    a = run_bwd_rab(case, dout, r)
    b = run_bwd_rab(case, dout, r)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("step", [3, 4, 64])
def test_rab_bwd_last_bucket_boundary(step):
    """Evenly spaced timestamps put the last-bucket boundary (gap 127 with 8
    buckets) a fixed number of keys below each query, so some 32-row blocks
    lie entirely in the last bucket and their neighbours do not; one time
    entry per bucket, well apart, makes a block misjudged either way show in
    dq, dk, dv and in the time table's gradient."""
    case, dout, r = make([300, 129, 64, 513], 2, 64, "bf16", 600, 8, seed=1570)
    r.timestamps = (np.arange(case.total, dtype=np.int64) * step).astype(np.int32)
    r.time_bias = (np.arange(8, dtype=np.float32) * np.float32(0.75) - np.float32(2.0))
    log(f"rab bwd last-bucket boundary, timestamp step {step}")
    compare(case, dout, r, run_bwd_rab(case, dout, r), f"rab bwd last bucket step {step}")
