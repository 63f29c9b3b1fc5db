"""Parity of the forward with the relative attention bias under the
target-aware mask against the fp64 CPU oracle, through the C ABI (HSTU paper
translation §3.4: M-FALCON adjusts the mask and rab_{p,t} together; the
reading, a candidate at the position right after the history with its own
timestamp, is the oracle's).

Small cases and the 16 x (3072 + 1024) ranking workload are compared element
by element (the workload also on sampled rows around the history/candidate
boundary through the oracle's row function).  Properties:
no candidates gives the causal bias forward bit for bit, and so does one
candidate per sequence (the last row is then its own candidate at its own
position); zero tables give the target-aware forward without bias bit for bit.
"""
import numpy as np
import pytest

import oracle
import workloads
from helpers import assert_close, device_case, from_torch, log

torch = pytest.importorskip("torch")
hstu = pytest.importorskip("generative_recommendation_attention_amd")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

# (length, candidates): t past either end (clamped), t = 0, 1, s - 1, s, and
# history/candidate boundaries on and around the 32-key blocks and the
# 128-row query tiles.
EDGE = [(1, 1), (2, 5), (31, 0), (32, 1), (33, 2), (63, 31), (64, 32), (65, 33),
        (127, 64), (128, 100), (129, 128), (255, 200), (256, 255), (257, 1), (383, 350),
        (0, 0), (511, 17), (3, -4), (300, 64), (200, 200), (450, 97), (97, 96)]


def make(pairs, heads, d, dtype, seed, npos, ntime, sigma=1.0, alpha=None, n=None):
    case = workloads.make_case([s for s, _ in pairs], heads, d, dtype, seed=seed, sigma=sigma,
                               alpha=alpha, n=n)
    case.num_targets = np.array([t for _, t in pairs], np.int32)
    return case, workloads.make_rab_inputs(case.offsets, npos, ntime, seed=seed + 1)


def bias_tensors(r):
    return (torch.from_numpy(r.timestamps).cuda(), torch.from_numpy(r.pos_bias).cuda(),
            torch.from_numpy(r.time_bias).cuda())


def run(case, r, num_targets=None):
    q, k, v, off = device_case(case)
    ts, wp, wt = bias_tensors(r)
    tg = case.num_targets if num_targets is None else num_targets
    res = hstu.hstu_attn_fwd_rab_targets(q, k, v, off, torch.from_numpy(tg).cuda(), ts, wp, wt,
                                         case.alpha, case.n)
    torch.cuda.synchronize()
    return res


def oracle_fwd(case, r):
    return oracle.fwd_rab(case.q, case.k, case.v, case.offsets, r.timestamps, r.pos_bias,
                          r.time_bias, case.heads, case.d, case.alpha, case.n, case.dtype,
                          num_targets=case.num_targets)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("npos,ntime", [(1000, 12), (70, 32)])
def test_rab_targets_full_compare(dtype, d, npos, ntime):
    case, r = make(EDGE, 2, d, dtype, seed=1500 + d + npos, npos=npos, ntime=ntime,
                   sigma=0.5 if dtype == "fp16" else 1.0)
    log(f"rab targets {dtype} d={d} npos={npos} ntime={ntime} T={case.total}")
    got = from_torch(run(case, r), dtype)
    mr, l2 = assert_close(got, oracle_fwd(case, r), dtype,
                          f"rab targets {dtype} d{d} npos{npos} ntime{ntime}")
    log(f"  max|err|/max|ref| = {mr:.3e}, rel L2 = {l2:.3e}")


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("fp16", 128), ("fp32", 64), ("bf16", 128)])
@pytest.mark.parametrize("t", [0, 1])
def test_zero_or_one_candidate_is_causal_rab_bitwise(dtype, d, t):
    pairs = [(s, t) for s in (1, 37, 300, 129, 0, 513, 64, 255)]
    case, r = make(pairs, 2, d, dtype, seed=1520, npos=600, ntime=16,
                   sigma=0.5 if dtype == "fp16" else 1.0)
    got = run(case, r)
    q, k, v, off = device_case(case)
    ts, wp, wt = bias_tensors(r)
    causal = hstu.hstu_attn_fwd_rab(q, k, v, off, ts, wp, wt, case.alpha, case.n)
    torch.cuda.synchronize()
    view = torch.int32 if dtype == "fp32" else torch.int16
    assert torch.equal(got.view(view), causal.view(view))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_zero_tables_match_targets_without_bias_bitwise(dtype):
    case, r = make(EDGE, 3, 64, dtype, seed=1530, npos=50, ntime=8)
    r.pos_bias[:] = 0
    r.time_bias[:] = 0
    got = run(case, r)
    q, k, v, off = device_case(case)
    plain = hstu.hstu_attn_fwd_targets(q, k, v, off, torch.from_numpy(case.num_targets).cuda(),
                                       case.alpha, case.n)
    torch.cuda.synchronize()
    view = torch.int32 if dtype == "fp32" else torch.int16
    assert torch.equal(got.view(view), plain.view(view))


def test_candidate_order_permutes_outputs():
    """Reversing each sequence's candidates (q, k, v and timestamps) reverses
    their output rows; the history rows stay as they were."""
    pairs = [(300, 64), (129, 128), (511, 17), (97, 96)]
    case, r = make(pairs, 2, 64, "bf16", seed=1540, npos=400, ntime=16)
    base = from_torch(run(case, r), "bf16")
    perm = np.arange(case.total)
    for i, (s, t) in enumerate(pairs):
        b = int(case.offsets[i + 1])
        perm[b - t:b] = perm[b - t:b][::-1]
    case2, r2 = make(pairs, 2, 64, "bf16", seed=1540, npos=400, ntime=16)
    case2.q, case2.k, case2.v = case.q[perm], case.k[perm], case.v[perm]
    r2.timestamps = r.timestamps[perm].copy()
    got = from_torch(run(case2, r2), "bf16")
    assert_close(got, base[perm], "bf16", "candidate order")


def test_rab_targets_many_sequences_worklist_path():
    """More than 256 sequences: the work list comes from the work-list kernel."""
    rng = np.random.default_rng(21)
    lengths = rng.integers(0, 160, size=300)
    tg = [int(rng.integers(0, s + 2)) for s in lengths]
    case, r = make(list(zip(lengths.tolist(), tg)), 2, 64, "bf16", seed=1550, npos=120,
                   ntime=10)
    got = from_torch(run(case, r), "bf16")
    assert_close(got, oracle_fwd(case, r), "bf16", "rab targets 300 sequences")


def test_rab_targets_workload_whole_output_and_sampled_rows():
    """16 x (3072 history + 1024 candidates), heads 4, d 64, bf16, a position
    entry per distance and 16 time buckets: the whole output, and rows on
    both sides of the history/candidate boundary, tile edges and random rows
    through the oracle's row function."""
    case, r = workloads.rab_targets_workload()
    log(f"rab targets workload: T={case.total}")
    out = run(case, r)
    rng = np.random.default_rng(12)
    rows = np.concatenate([[0, 127, 3071, 3072, 3073, 3199, 3200, 4095],
                           rng.integers(0, 4096, size=8)])
    seqs = rng.integers(0, 16, size=len(rows))
    tok = (seqs * 4096 + rows).astype(np.int64)
    hd = rng.integers(0, 4, size=len(tok)).astype(np.int32)
    got = from_torch(out[torch.from_numpy(tok).cuda(), torch.from_numpy(hd).cuda()], "bf16")
    ref = oracle.rows_rab(case.q, case.k, case.v, case.offsets, r.timestamps, r.pos_bias,
                          r.time_bias, 4, 64, case.alpha, case.n, "bf16", tok, hd,
                          num_targets=case.num_targets)
    mr, l2 = assert_close(got, ref, "bf16", "rab targets workload rows")
    log(f"  max|err|/max|ref| = {mr:.3e}, rel L2 = {l2:.3e}")
    mr, l2 = assert_close(from_torch(out, "bf16"), oracle_fwd(case, r), "bf16",
                          "rab targets workload whole output")
    log(f"  whole output: max|err|/max|ref| = {mr:.3e}, rel L2 = {l2:.3e}")
    assert torch.isfinite(out.float()).all().item()


def test_rab_targets_binding_rejects_bad_counts():
    case, r = make([(10, 2), (5, 1)], 1, 64, "bf16", seed=1, npos=8, ntime=4)
    q, k, v, off = device_case(case)
    ts, wp, wt = bias_tensors(r)
    with pytest.raises(ValueError):
        hstu.hstu_attn_fwd_rab_targets(q, k, v, off, torch.zeros(3, dtype=torch.int32).cuda(),
                                       ts, wp, wt, 0.1, 1.0)
    with pytest.raises(ValueError):
        hstu.hstu_attn_fwd_rab_targets(q, k, v, off, torch.zeros(2, dtype=torch.int32).cuda(),
                                       ts[:3], wp, wt, 0.1, 1.0)
