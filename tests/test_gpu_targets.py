"""Parity of the target-aware (M-FALCON) forward against the fp64 CPU oracle,
through the C ABI (HSTU paper translation §3.4, Appendix H, Fig. 11: the last
t tokens of a sequence are candidates that see the history and themselves).

Small cases are compared element by element; the 16 x (3072 + 1024) ranking
workload element by element too, and on sampled rows around the
history/candidate boundary through the oracle's row function.
Properties: t = 0 and t = 1 give the plain causal result bit for bit, history
rows are untouched by the candidates, and each candidate's row equals the
plain causal result of its history followed by that candidate alone.
"""
import numpy as np
import pytest

import oracle
import workloads
from helpers import assert_close, device_case, errors, from_torch, log, TOL

torch = pytest.importorskip("torch")
hstu = pytest.importorskip("generative_recommendation_attention_amd")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

# Lengths and candidate counts: t past either end (clamped), t = 0, 1, s-1, s,
# and history/candidate boundaries on and around the 32-key blocks and the
# query tiles.
EDGE = [(1, 1), (2, 5), (31, 0), (32, 1), (33, 2), (63, 31), (64, 32), (65, 33),
        (127, 64), (128, 100), (129, 128), (255, 200), (256, 255), (257, 1), (383, 350),
        (0, 0), (511, 17), (3, -4), (300, 64), (200, 200), (450, 97), (97, 96)]


def targets_case(pairs, heads, d, dtype, seed, sigma=1.0, alpha=None, n=None):
    lengths = [s for s, _ in pairs]
    case = workloads.make_case(lengths, heads, d, dtype, seed=seed, sigma=sigma, alpha=alpha,
                               n=n)
    case.num_targets = np.array([t for _, t in pairs], np.int32)
    return case


def run_targets(case, out=None):
    q, k, v, off = device_case(case)
    tg = torch.from_numpy(case.num_targets.astype(np.int32)).cuda()
    res = hstu.hstu_attn_fwd_targets(q, k, v, off, tg, case.alpha, case.n, out=out)
    torch.cuda.synchronize()
    return res


def run_plain(case):
    q, k, v, off = device_case(case)
    res = hstu.hstu_attn_fwd(q, k, v, off, case.alpha, case.n)
    torch.cuda.synchronize()
    return res


def oracle_fwd(case):
    return oracle.fwd(case.q, case.k, case.v, case.offsets, case.heads, case.d, case.alpha,
                      case.n, case.dtype, num_targets=case.num_targets)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
def test_targets_edge_full_compare(dtype, d):
    case = targets_case(EDGE, 2, d, dtype, seed=500 + d,
                        sigma=0.5 if dtype == "fp16" else 1.0, alpha=1.0 / np.sqrt(d), n=511.0)
    log(f"targets edge {dtype} d={d} T={case.total}")
    got = from_torch(run_targets(case), dtype)
    ref = oracle_fwd(case)
    assert_close(got, ref, dtype, f"targets edge {dtype} d{d}")
    for i in range(case.num_seqs):
        a, b = int(case.offsets[i]), int(case.offsets[i + 1])
        if b > a:
            mr, l2 = errors(got[a:b], ref[a:b])
            assert mr <= TOL[dtype][0] * 2 and l2 <= TOL[dtype][1] * 2, (i, EDGE[i], mr, l2)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_targets_many_sequences_two_kernel_form(dtype):
    """More sequences than the one-kernel form takes: the work-list kernel runs."""
    rng = np.random.default_rng(17)
    lengths = rng.integers(0, 200, size=300)
    tg = [int(rng.integers(-2, s + 3)) for s in lengths]
    case = targets_case(list(zip(lengths.tolist(), tg)), 3, 64, dtype, seed=521, alpha=0.1,
                        n=200.0)
    log(f"targets many sequences {dtype} T={case.total}")
    got = from_torch(run_targets(case), dtype)
    assert_close(got, oracle_fwd(case), dtype, f"targets 300 seqs {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_zero_or_one_candidate_is_plain_causal(dtype):
    """A sequence whose only candidate is its last token, or that has none, has
    the plain causal mask: the results agree bit for bit."""
    rng = np.random.default_rng(23)
    lengths = rng.integers(1, 700, size=24).tolist()
    pairs = [(s, int(i % 2)) for i, s in enumerate(lengths)]
    case = targets_case(pairs, 2, 64 if dtype != "fp16" else 128, dtype, seed=531,
                        sigma=0.5 if dtype == "fp16" else 1.0, alpha=0.125, n=700.0)
    log(f"t in (0, 1) vs plain {dtype}")
    a = run_targets(case)
    b = run_plain(case)
    assert torch.equal(a.view(torch.int16) if dtype != "fp32" else a.view(torch.int32),
                       b.view(torch.int16) if dtype != "fp32" else b.view(torch.int32))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_history_rows_match_plain_causal(dtype):
    """Rows before the first candidate see only earlier history keys, so they
    agree bit for bit with the plain causal call (keys are accumulated in the
    same ascending block order either way)."""
    rng = np.random.default_rng(29)
    lengths = rng.integers(40, 900, size=20).tolist()
    pairs = [(s, int(rng.integers(0, s + 1))) for s in lengths]
    case = targets_case(pairs, 4, 64, dtype, seed=541, alpha=0.125, n=900.0)
    log(f"history rows vs plain {dtype}")
    a = from_torch(run_targets(case), dtype)
    b = from_torch(run_plain(case), dtype)
    for i, (s, t) in enumerate(pairs):
        h = s - min(max(t, 0), s)
        lo = int(case.offsets[i])
        assert np.array_equal(a[lo:lo + h], b[lo:lo + h]), (i, s, t)


def test_candidates_equal_separate_passes():
    """M-FALCON's claim (Appendix H): one pass over history + b_m candidates
    gives each candidate the result of a causal pass over history + that
    candidate alone.  Both sides run on the GPU; the separate passes are a
    plain causal batch of b_m sequences."""
    rng = np.random.default_rng(31)
    h, bm, heads, d = 700, 45, 2, 64
    big = targets_case([(h + bm, bm)], heads, d, "bf16", seed=551, alpha=0.125, n=745.0)
    out = from_torch(run_targets(big), "bf16")
    # b_m sequences of h + 1 tokens: the history, then candidate j.
    sep = workloads.make_case([h + 1] * bm, heads, d, "bf16", seed=0, alpha=0.125, n=745.0)
    for name in ("q", "k", "v"):
        src = getattr(big, name)
        dst = np.concatenate([np.concatenate([src[:h], src[h + j:h + j + 1]]) for j in range(bm)])
        setattr(sep, name, dst)
    sout = from_torch(run_plain(sep), "bf16")
    cand_sep = sout.reshape(bm, h + 1, heads, d)[:, h]
    cand_big = out[h:h + bm]
    mr, l2 = errors(cand_big, cand_sep)
    log(f"  candidates vs separate passes: {mr:.3e} {l2:.3e}")
    assert mr <= TOL["bf16"][0] and l2 <= TOL["bf16"][1]
    del rng


def sample_target_rows(case, seed=11, per_seq_random=8):
    rng = np.random.default_rng(seed)
    toks, hds = [], []
    for i in range(case.num_seqs):
        s = int(case.lengths[i])
        if s == 0:
            continue
        t = min(max(int(case.num_targets[i]), 0), s)
        h = s - t
        rows = {0, s - 1, h - 1, h, h + 1, h + 31, h + 32, h + 63, h + 64, s - 2}
        for b in (32, 64, 128, 256):
            rows |= {b - 1, b, b + 1}
        rows |= set(rng.integers(0, s, size=per_seq_random).tolist())
        rows = sorted(r for r in rows if 0 <= r < s)
        base = int(case.offsets[i])
        for r in rows:
            for hd in range(case.heads):
                toks.append(base + r)
                hds.append(hd)
    return np.array(toks, np.int64), np.array(hds, np.int32)


def test_targets_workload_whole_output_and_sampled_rows():
    case = workloads.targets_workload()
    log(f"targets workload: {case.description}; T={case.total}")
    got = run_targets(case)
    tok, hd = sample_target_rows(case)
    log(f"  checking {len(tok)} sampled rows")
    g = from_torch(got[torch.from_numpy(tok).cuda(), torch.from_numpy(hd.astype(np.int64)).cuda()],
                   case.dtype)
    ref = oracle.rows(case.q, case.k, case.v, case.offsets, case.heads, case.d, case.alpha,
                      case.n, case.dtype, tok, hd, num_targets=case.num_targets)
    mr, l2 = assert_close(g, ref, case.dtype, "targets workload sampled")
    log(f"  max|err|/max|ref| = {mr:.3e}, rel L2 = {l2:.3e}")
    mr, l2 = assert_close(from_torch(got, case.dtype), oracle_fwd(case), case.dtype,
                          "targets workload whole output")
    log(f"  whole output: max|err|/max|ref| = {mr:.3e}, rel L2 = {l2:.3e}")
    assert torch.isfinite(got.float()).all().item()


def test_targets_binding_rejects_bad_counts():
    case = targets_case([(10, 2), (5, 1)], 1, 64, "bf16", seed=1)
    q, k, v, off = device_case(case)
    with pytest.raises(ValueError):
        hstu.hstu_attn_fwd_targets(q, k, v, off, torch.zeros(3, dtype=torch.int32).cuda(),
                                   0.1, 1.0)
    with pytest.raises(ValueError):
        hstu.hstu_attn_fwd_targets(q, k, v, off, torch.zeros(2, dtype=torch.int64).cuda(),
                                   0.1, 1.0)
