"""Parity of the forward with the relative attention bias against the fp64
CPU oracle, through the C ABI (HSTU paper translation §3: rab_{p,t} is added
to the scores before SiLU; Appendix G: it is built inside the operator from
its parameters; the reading of the lost equation is the oracle's).

Small cases and the 16 x 4096 workload are compared element by element (the
workload also on sampled rows through the oracle's row function).  Properties: zero tables give the plain causal result bit for bit (the
bias only sets the score accumulators' initial value), and a bias that does
not depend on the pair shifts every score like one more head dimension.
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

# Lengths spanning several 32-key blocks, key tiles and 128-row query tiles,
# with ragged tails and an empty sequence.
LENGTHS = [1, 37, 300, 129, 0, 513, 64, 255]


def run_rab(case, r, out=None):
    q, k, v, off = device_case(case)
    ts = torch.from_numpy(r.timestamps).cuda()
    wp = torch.from_numpy(r.pos_bias).cuda()
    wt = torch.from_numpy(r.time_bias).cuda()
    res = hstu.hstu_attn_fwd_rab(q, k, v, off, ts, wp, wt, case.alpha, case.n, out=out)
    torch.cuda.synchronize()
    return res


def oracle_rab(case, r):
    return oracle.fwd_rab(case.q, case.k, case.v, case.offsets, r.timestamps, r.pos_bias,
                          r.time_bias, case.heads, case.d, case.alpha, case.n, case.dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("npos,ntime", [(1000, 12), (70, 32), (1, 1)])
def test_rab_full_compare(dtype, d, npos, ntime):
    case = workloads.make_case(LENGTHS, 2, d, dtype, seed=1400 + d + npos,
                               sigma=0.5 if dtype == "fp16" else 1.0)
    r = workloads.make_rab_inputs(case.offsets, npos, ntime, seed=1401 + ntime)
    log(f"rab {dtype} d={d} npos={npos} ntime={ntime} lengths={LENGTHS}")
    got = from_torch(run_rab(case, r), dtype)
    ref = oracle_rab(case, r)
    mr, l2 = assert_close(got, ref, dtype, f"rab {dtype} d{d} npos{npos} ntime{ntime}")
    log(f"  max|err|/max|ref| = {mr:.3e}, rel L2 = {l2:.3e}")


@pytest.mark.parametrize("kind", ["equal", "decreasing", "huge_gaps"])
def test_rab_timestamp_edges(kind):
    """Every gap 0 (bucket 0); timestamps running backwards (negative gaps:
    the last bucket); gaps near 2^30 (the cap)."""
    case = workloads.make_case([200, 77, 1], 2, 64, "bf16", seed=1410)
    r = workloads.make_rab_inputs(case.offsets, 150, 20, seed=1411)
    T = case.total
    if kind == "equal":
        r.timestamps = np.full(T, 123456, np.int32)
    elif kind == "decreasing":
        r.timestamps = (1_000_000 - 7 * np.arange(T)).astype(np.int32)
    else:
        r.timestamps = np.minimum(np.arange(T, dtype=np.int64) * (1 << 22), (1 << 31) - 2) \
            .astype(np.int32)
        r.timestamps[200:] -= r.timestamps[200]
    log(f"rab timestamps {kind}")
    got = from_torch(run_rab(case, r), "bf16")
    assert_close(got, oracle_rab(case, r), "bf16", f"rab timestamps {kind}")


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("fp16", 128), ("fp32", 64)])
def test_rab_zero_tables_match_plain_bitwise(dtype, d):
    case = workloads.make_case(LENGTHS + [700], 3, d, dtype, seed=1420,
                               sigma=0.5 if dtype == "fp16" else 1.0)
    r = workloads.make_rab_inputs(case.offsets, 40, 8, seed=1421)
    r.pos_bias[:] = 0
    r.time_bias[:] = 0
    got = run_rab(case, r)
    q, k, v, off = device_case(case)
    plain = hstu.hstu_attn_fwd(q, k, v, off, case.alpha, case.n)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16 if dtype != "fp32" else torch.int32),
                       plain.view(torch.int16 if dtype != "fp32" else torch.int32))


def test_rab_constant_bias_is_one_more_dimension():
    """wpos = beta everywhere inside the table, wtime = 0: each score grows by
    beta, which is alpha <[q, 1], [k, beta / alpha]> (fp32, d 64 + 1 in the
    oracle's plain forward)."""
    case = workloads.make_case([90, 257, 33], 2, 64, "fp32", seed=1430, alpha=0.125, n=257.0)
    r = workloads.make_rab_inputs(case.offsets, 300, 4, seed=1431)
    r.pos_bias[:] = np.float32(0.25)
    r.time_bias[:] = 0
    got = from_torch(run_rab(case, r), "fp32")
    T, H, d = case.q.shape
    q = np.concatenate([case.q, np.ones((T, H, 1), np.float32)], axis=2)
    k = np.concatenate([case.k, np.full((T, H, 1), 2.0, np.float32)], axis=2)
    v = np.concatenate([case.v, np.zeros((T, H, 1), np.float32)], axis=2)
    ref = oracle.fwd(q, k, v, case.offsets, H, d + 1, case.alpha, case.n, "fp32")[:, :, :d]
    assert_close(got, ref, "fp32", "rab constant bias")


def test_rab_many_sequences_worklist_path():
    """More than 256 sequences: the work list comes from the work-list kernel."""
    lengths = list(np.random.default_rng(3).integers(0, 140, size=300))
    case = workloads.make_case(lengths, 2, 64, "bf16", seed=1440)
    r = workloads.make_rab_inputs(case.offsets, 100, 10, seed=1441)
    got = from_torch(run_rab(case, r), "bf16")
    assert_close(got, oracle_rab(case, r), "bf16", "rab 300 sequences")


def test_rab_workload_whole_output_and_sampled_rows():
    """16 x 4096, heads 4, d 64, bf16, a position entry per distance and 16
    time buckets: the whole output, and sampled rows (tile edges and random)
    of every head through the oracle's row function."""
    case, r = workloads.rab_workload()
    log("rab workload 16 x 4096 (whole output and sampled rows)")
    out = run_rab(case, r)
    rng = np.random.default_rng(11)
    seqs = rng.integers(0, 16, size=24)
    rows = np.concatenate([[0, 31, 32, 127, 128, 4095], rng.integers(0, 4096, size=18)])
    tok = (seqs * 4096 + rows).astype(np.int64)
    hd = rng.integers(0, 4, size=len(tok)).astype(np.int32)
    got = from_torch(out[torch.from_numpy(tok).cuda(), torch.from_numpy(hd).cuda()], "bf16")
    ref = oracle.rows_rab(case.q, case.k, case.v, case.offsets, r.timestamps, r.pos_bias,
                          r.time_bias, 4, 64, case.alpha, case.n, "bf16", tok, hd)
    mr, l2 = assert_close(got, ref, "bf16", "rab workload rows")
    log(f"  max|err|/max|ref| = {mr:.3e}, rel L2 = {l2:.3e}")
    mr, l2 = assert_close(from_torch(out, "bf16"), oracle_rab(case, r), "bf16",
                          "rab workload whole output")
    log(f"  whole output: max|err|/max|ref| = {mr:.3e}, rel L2 = {l2:.3e}")


def test_rab_repeat_is_deterministic():
    case = workloads.make_case([1000, 300], 4, 64, "bf16", seed=1450)
    r = workloads.make_rab_inputs(case.offsets, 500, 16, seed=1451)
    a = run_rab(case, r)
    b = run_rab(case, r)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("step", [3, 4, 5, 64])
def test_rab_last_bucket_boundary(step):
    """Evenly spaced timestamps put the last-bucket boundary (gap
    2^(ntime-1) - 1 = 127 with 8 buckets) a fixed number of keys below each
    row, so some 32-key blocks lie entirely in the last bucket and their
    neighbours do not; with one time entry per bucket well apart, a block
    given the constant last-bucket term by mistake would show."""
    case = workloads.make_case([300, 129, 64, 513], 2, 64, "bf16", seed=1460)
    r = workloads.make_rab_inputs(case.offsets, 600, 8, seed=1461)
    r.timestamps = (np.arange(case.total, dtype=np.int64) * step).astype(np.int32)
    r.time_bias = (np.arange(8, dtype=np.float32) * np.float32(0.75) - np.float32(2.0))
    log(f"rab last-bucket boundary, timestamp step {step}")
    got = from_torch(run_rab(case, r), "bf16")
    assert_close(got, oracle_rab(case, r), "bf16", f"rab last bucket step {step}")
