"""Parity of the backward with the relative attention bias under the
target-aware mask against the fp64 CPU oracle, through the C ABI (HSTU paper
translation §3.4: M-FALCON changes the mask and rab_{p,t} together;
Appendix G: the bias gradients are accumulated on chip).  The oracle's
reading: a candidate row sits right after the history (distance hist - c to
a history key, 0 to itself) and keeps its own timestamp; a pair's score
gradient goes to the entries its bias used.

dq, dk, dv and both table gradients are compared element by element on cases
whose candidates start on and around 32-key blocks and 128-row tiles, fill
whole tiles (the dQ kernel then jumps over candidate-only key blocks) and
reach past a short position table.  The table gradients are float sums taken
with atomics, so they are compared within the tolerance.  Properties: no
candidate, or one, gives the causal bias backward's dq, dk, dv bit for bit;
zero tables give the target-aware backward without bias bit for bit.  The
16 x (3072 + 1024) ranking workload: every element, and equal table totals.
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

# (length, candidates): t clamped past either end, t = 0, 1, s - 1, s, and
# history/candidate boundaries on and around 32-key blocks and 128-row tiles;
# (600, 400) and (520, 500) put several whole query tiles past the history.
EDGE = [(1, 1), (2, 5), (31, 0), (33, 2), (64, 32), (65, 33), (127, 64), (129, 128),
        (256, 255), (257, 1), (0, 0), (300, 64), (200, 200), (450, 97), (97, 96), (3, -4),
        (600, 400), (520, 500)]


def make(pairs, heads, d, dtype, seed, npos, ntime):
    sigma = 0.5 if dtype == "fp16" else 1.0
    lengths = [s for s, _ in pairs]
    case = workloads.make_case(lengths, heads, d, dtype, seed=seed, sigma=sigma)
    case.num_targets = np.array([t for _, t in pairs], np.int32)
    dout = workloads.make_case(lengths, heads, d, dtype, seed=seed + 1, sigma=sigma).q
    r = workloads.make_rab_inputs(case.offsets, npos, ntime, seed=seed + 2)
    return case, dout, r


def bias_tensors(r):
    return (torch.from_numpy(r.timestamps).cuda(), torch.from_numpy(r.pos_bias).cuda(),
            torch.from_numpy(r.time_bias).cuda())


def run(case, dout, r, num_targets=None):
    q, k, v, off = device_case(case)
    ts, wp, wt = bias_tensors(r)
    tg = case.num_targets if num_targets is None else num_targets
    res = hstu.hstu_attn_bwd_rab_targets(q, k, v, to_torch(dout, case.dtype), off,
                                         torch.from_numpy(tg).cuda(), ts, wp, wt, case.alpha,
                                         case.n)
    torch.cuda.synchronize()
    return res


def compare(case, dout, r, res, what):
    ref = oracle.bwd_rab(case.q, case.k, case.v, dout, case.offsets, r.timestamps, r.pos_bias,
                         r.time_bias, case.heads, case.d, case.alpha, case.n, case.dtype,
                         num_targets=case.num_targets)
    for name, g, rf in zip(("dq", "dk", "dv"), res[:3], ref[:3]):
        assert_close(from_torch(g, case.dtype), rf, case.dtype, f"{what} {name}")
    for name, g, rf in zip(("d_pos_bias", "d_time_bias"), res[3:], ref[3:]):
        mr, l2 = assert_close(g.cpu().numpy().astype(np.float64), rf, case.dtype,
                              f"{what} {name}")
        log(f"  {name}: max|err|/max|ref| = {mr:.2e}, rel L2 = {l2:.2e}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("npos,ntime", [(700, 16), (40, 32)])
def test_rab_bwd_targets_full_compare(dtype, d, npos, ntime):
    case, dout, r = make(EDGE, 2, d, dtype, seed=1600 + d + npos, npos=npos, ntime=ntime)
    log(f"rab bwd targets {dtype} d={d} npos={npos} ntime={ntime}")
    compare(case, dout, r, run(case, dout, r), f"rab bwd targets {dtype} d{d}")


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("fp16", 128), ("fp32", 64)])
@pytest.mark.parametrize("t", [0, 1])
def test_zero_or_one_candidate_is_causal_bitwise(dtype, d, t):
    """dq, dk, dv equal the causal bias backward's bit for bit (one candidate
    is the last row, already at distance s - 1 - c from every key); the table
    gradients agree within the tolerance (they are summed in another order)."""
    pairs = [(s, t) for s in (1, 37, 300, 129, 200, 64, 513)]
    case, dout, r = make(pairs, 3, d, dtype, seed=1620 + t, npos=300, ntime=12)
    got = run(case, dout, r)
    q, k, v, off = device_case(case)
    ts, wp, wt = bias_tensors(r)
    causal = hstu.hstu_attn_bwd_rab(q, k, v, to_torch(dout, dtype), off, ts, wp, wt, case.alpha,
                                    case.n)
    torch.cuda.synchronize()
    view = torch.int32 if dtype == "fp32" else torch.int16
    for a, b in zip(got[:3], causal[:3]):
        assert torch.equal(a.view(view), b.view(view))
    for a, b in zip(got[3:], causal[3:]):
        assert_close(a.cpu().numpy().astype(np.float64), b.cpu().numpy().astype(np.float64),
                     dtype, "tables")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_zero_tables_match_targets_without_bias_bitwise(dtype):
    case, dout, r = make(EDGE, 2, 64, dtype, seed=1630, npos=50, ntime=6)
    r.pos_bias[:] = 0
    r.time_bias[:] = 0
    got = run(case, dout, r)
    q, k, v, off = device_case(case)
    plain = hstu.hstu_attn_bwd(q, k, v, to_torch(dout, dtype), off, case.alpha, case.n,
                               num_targets=torch.from_numpy(case.num_targets).cuda())
    torch.cuda.synchronize()
    view = torch.int32 if dtype == "fp32" else torch.int16
    for a, b in zip(got[:3], plain):
        assert torch.equal(a.view(view), b.view(view))
    assert float(got[3].abs().sum()) > 0 and float(got[4].abs().sum()) > 0


def test_rab_bwd_targets_many_sequences_worklist_path():
    """More than 256 sequences: the work list comes from the work-list kernel."""
    rng = np.random.default_rng(22)
    lengths = rng.integers(0, 200, size=300)
    tg = [int(rng.integers(0, s + 2)) for s in lengths]
    case, dout, r = make(list(zip(lengths.tolist(), tg)), 2, 64, "bf16", seed=1640, npos=150,
                         ntime=10)
    compare(case, dout, r, run(case, dout, r), "rab bwd targets 300 sequences")


def test_rab_bwd_targets_mid_size_full_compare():
    """4 users x (700 history + 300 candidates), heads 2, d 64, bf16, a
    position entry per distance: every gradient element by element."""
    case, dout, r = make([(1000, 300)] * 4, 2, 64, "bf16", seed=1650, npos=1000, ntime=16)
    log("rab bwd targets 4 x (700 + 300)")
    compare(case, dout, r, run(case, dout, r), "rab bwd targets 4 x 1000")


def test_rab_bwd_targets_workload_full_compare_and_totals():
    """16 x (3072 history + 1024 candidates), heads 4, d 64, bf16, a position
    entry per distance and 16 time buckets: every element of dq, dk, dv and
    of both table gradients against the oracle (about 45 s of oracle time on
    16 host threads), and equal totals of the two table gradients."""
    case, r = workloads.rab_targets_workload()
    dout = workloads.make_case([4096] * 16, 4, 64, "bf16", seed=1660).q
    log(f"rab bwd targets workload: T={case.total} (whole output)")
    res = run(case, dout, r)
    ref = oracle.bwd_rab(case.q, case.k, case.v, dout, case.offsets, r.timestamps, r.pos_bias,
                         r.time_bias, 4, 64, case.alpha, case.n, "bf16",
                         num_targets=case.num_targets)
    for name, g, rf in zip(("dq", "dk", "dv"), res[:3], ref[:3]):
        mr, l2 = assert_close(from_torch(g, "bf16"), rf, "bf16", f"rab bwd targets workload {name}")
        log(f"  {name}: max|err|/max|ref| = {mr:.2e}, rel L2 = {l2:.2e}")
    for name, g, rf in zip(("d_pos_bias", "d_time_bias"), res[3:], ref[3:]):
        mr, l2 = assert_close(g.cpu().numpy().astype(np.float64), rf, "bf16",
                              f"rab bwd targets workload {name}")
        log(f"  {name}: max|err|/max|ref| = {mr:.2e}, rel L2 = {l2:.2e}")
    sp = float(res[3].double().sum())
    st = float(res[4].double().sum())
    scale = float(res[3].double().abs().sum())
    assert abs(sp - st) <= 1e-4 * scale, (sp, st, scale)


def test_rab_bwd_targets_binding_rejects_bad_counts():
    case, dout, r = make([(10, 2), (5, 1)], 1, 64, "bf16", seed=1, npos=8, ntime=4)
    q, k, v, off = device_case(case)
    ts, wp, wt = bias_tensors(r)
    do = to_torch(dout, "bf16")
    with pytest.raises(ValueError):
        hstu.hstu_attn_bwd_rab_targets(q, k, v, do, off, torch.zeros(3, dtype=torch.int32).cuda(),
                                       ts, wp, wt, 0.1, 1.0)
