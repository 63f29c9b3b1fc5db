"""Parity of the cached-history forward (M-FALCON's later micro-batches, HSTU
paper translation Appendix H) against the fp64 CPU oracle, through the C ABI.

Candidates with their own q, k, v attend to a cached history's K and V plus
themselves.  Small cases are compared element by element; the 16 x (3072
cached + 1024 candidates) workload element by element too, and on sampled
rows through the oracle's row function.  Properties: the result
equals the candidate rows of one target-aware pass over history + candidates
(GPU against GPU, within tolerance), and a request without history gives
each candidate silu(alpha <q, k>) v / n.
"""
import numpy as np
import pytest

import oracle
import workloads
from helpers import TOL, assert_close, errors, from_torch, log, to_torch

torch = pytest.importorskip("torch")
hstu = pytest.importorskip("generative_recommendation_attention_amd")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

# (history rows, candidates): empty history, empty micro-batch, history on
# and around key-tile edges (32 and 64 keys), candidates across Q tiles.
EDGE = [(0, 5), (1, 1), (31, 2), (32, 33), (33, 64), (63, 1), (64, 100), (65, 128),
        (100, 0), (127, 129), (128, 255), (129, 256), (300, 257), (511, 31), (0, 0),
        (2, 300), (97, 3), (256, 1)]


def device(cc: workloads.CachedCase):
    c = cc.cand
    dt = c.dtype
    return (to_torch(c.q, dt), to_torch(c.k, dt), to_torch(c.v, dt),
            torch.from_numpy(c.offsets.astype(np.int32)).cuda(),
            to_torch(cc.k_cache, dt), to_torch(cc.v_cache, dt),
            torch.from_numpy(cc.hist_offsets.astype(np.int32)).cuda())


def run_cached(cc, out=None):
    q, k, v, coff, kc, vc, hoff = device(cc)
    res = hstu.hstu_attn_fwd_cached(q, k, v, coff, kc, vc, hoff, cc.cand.alpha, cc.cand.n,
                                    out=out)
    torch.cuda.synchronize()
    return res


def oracle_cached(cc):
    c = cc.cand
    return oracle.fwd_cached(c.q, c.k, c.v, c.offsets, cc.k_cache, cc.v_cache,
                             cc.hist_offsets, c.heads, c.d, c.alpha, c.n, c.dtype)


def edge_case(dtype, d, seed):
    return workloads.make_cached_case([h for h, _ in EDGE], [t for _, t in EDGE], 2, d, dtype,
                                      seed=seed, sigma=0.5 if dtype == "fp16" else 1.0,
                                      alpha=1.0 / np.sqrt(d), n=811.0)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
def test_cached_edge_full_compare(dtype, d):
    cc = edge_case(dtype, d, seed=600 + d)
    log(f"cached edge {dtype} d={d} Tc={cc.cand.total} Th={int(cc.hist_offsets[-1])}")
    got = from_torch(run_cached(cc), dtype)
    ref = oracle_cached(cc)
    assert_close(got, ref, dtype, f"cached edge {dtype} d{d}")
    off = cc.cand.offsets
    for i in range(cc.cand.num_seqs):
        a, b = int(off[i]), int(off[i + 1])
        if b > a:
            mr, l2 = errors(got[a:b], ref[a:b])
            assert mr <= TOL[dtype][0] * 2 and l2 <= TOL[dtype][1] * 2, (i, EDGE[i], mr, l2)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_cached_many_requests_two_kernel_form(dtype):
    """More requests than the one-kernel form takes: the work-list kernel runs."""
    rng = np.random.default_rng(19)
    hist = rng.integers(0, 150, size=300).tolist()
    cand = rng.integers(0, 90, size=300).tolist()
    cc = workloads.make_cached_case(hist, cand, 3, 64, dtype, seed=611, alpha=0.1, n=240.0)
    log(f"cached 300 requests {dtype} Tc={cc.cand.total}")
    got = from_torch(run_cached(cc), dtype)
    assert_close(got, oracle_cached(cc), dtype, f"cached 300 requests {dtype}")


def test_cached_equals_one_target_aware_pass():
    """The cached form gives the candidates what one pass over history +
    candidates with the target-aware mask gives them (both on the GPU)."""
    hist, cand = [700, 64, 0, 129], [45, 200, 7, 64]
    cc = workloads.make_cached_case(hist, cand, 2, 64, "bf16", seed=621, alpha=0.125, n=900.0)
    got = from_torch(run_cached(cc), "bf16")
    c = cc.cand
    qs, ks, vs, lens = [], [], [], []
    for i in range(c.num_seqs):
        ha, hb = int(cc.hist_offsets[i]), int(cc.hist_offsets[i + 1])
        ca, cb = int(c.offsets[i]), int(c.offsets[i + 1])
        qs += [np.zeros_like(cc.k_cache[ha:hb]), c.q[ca:cb]]
        ks += [cc.k_cache[ha:hb], c.k[ca:cb]]
        vs += [cc.v_cache[ha:hb], c.v[ca:cb]]
        lens.append(hb - ha + cb - ca)
    off = workloads.offsets_from_lengths(lens)
    q, k, v = (to_torch(np.concatenate(x), "bf16") for x in (qs, ks, vs))
    full = hstu.hstu_attn_fwd_targets(q, k, v, torch.from_numpy(off).cuda(),
                                      torch.tensor(cand, dtype=torch.int32).cuda(),
                                      c.alpha, c.n)
    full = from_torch(full, "bf16")
    ref = np.concatenate([full[int(off[i]) + hist[i]:int(off[i + 1])] for i in range(len(hist))])
    mr, l2 = errors(got, ref)
    log(f"  cached vs one pass: {mr:.3e} {l2:.3e}")
    assert mr <= TOL["bf16"][0] and l2 <= TOL["bf16"][1]


def test_cached_without_history_closed_form():
    cc = workloads.make_cached_case([0, 0, 0], [70, 1, 300], 4, 128, "fp32", seed=631,
                                    alpha=0.09, n=3.0)
    got = from_torch(run_cached(cc), "fp32")
    c = cc.cand
    q, k, v = (oracle.widen(x, "fp32") for x in (c.q, c.k, c.v))
    x = c.alpha * np.sum(q * k, axis=-1, keepdims=True)
    ref = x / (1.0 + np.exp(-x)) * v / c.n
    assert_close(got, ref, "fp32", "cached, no history")


def sample_cached_rows(cc, seed=13, per_seq_random=8):
    rng = np.random.default_rng(seed)
    toks, hds = [], []
    c = cc.cand
    for i in range(c.num_seqs):
        t = int(c.lengths[i])
        if t == 0:
            continue
        rows = {0, 1, 31, 32, 63, 64, 127, 128, 255, 256, t - 1, t - 2}
        rows |= set(rng.integers(0, t, size=per_seq_random).tolist())
        base = int(c.offsets[i])
        for r in sorted(r for r in rows if 0 <= r < t):
            for hd in range(c.heads):
                toks.append(base + r)
                hds.append(hd)
    return np.array(toks, np.int64), np.array(hds, np.int32)


def test_cached_workload_whole_output_and_sampled_rows():
    cc = workloads.cached_workload()
    c = cc.cand
    log(f"cached workload: {c.description}")
    got = run_cached(cc)
    tok, hd = sample_cached_rows(cc)
    log(f"  checking {len(tok)} sampled rows")
    g = from_torch(got[torch.from_numpy(tok).cuda(), torch.from_numpy(hd.astype(np.int64)).cuda()],
                   c.dtype)
    ref = oracle.rows_cached(c.q, c.k, c.v, c.offsets, cc.k_cache, cc.v_cache, cc.hist_offsets,
                             c.heads, c.d, c.alpha, c.n, c.dtype, tok, hd)
    mr, l2 = assert_close(g, ref, c.dtype, "cached workload sampled")
    log(f"  max|err|/max|ref| = {mr:.3e}, rel L2 = {l2:.3e}")
    mr, l2 = assert_close(from_torch(got, c.dtype), oracle_cached(cc), c.dtype,
                          "cached workload whole output")
    log(f"  whole output: max|err|/max|ref| = {mr:.3e}, rel L2 = {l2:.3e}")
    assert torch.isfinite(got.float()).all().item()


def test_cached_binding_rejects_bad_inputs():
    cc = workloads.make_cached_case([3, 2], [2, 1], 1, 64, "bf16", seed=1)
    q, k, v, coff, kc, vc, hoff = device(cc)
    with pytest.raises(ValueError):   # history offsets of the wrong length
        hstu.hstu_attn_fwd_cached(q, k, v, coff, kc, vc, hoff[:2], 0.1, 1.0)
    with pytest.raises(ValueError):   # cache of another head size
        hstu.hstu_attn_fwd_cached(q, k, v, coff, kc[:, :, :32].contiguous(), vc, hoff, 0.1, 1.0)
    with pytest.raises(ValueError):   # cache of another element type
        hstu.hstu_attn_fwd_cached(q, k, v, coff, kc.half(), vc, hoff, 0.1, 1.0)


def test_cached_empty_inputs():
    """No candidates at all, and no history at all (empty cache tensors)."""
    z = torch.zeros((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    coff = torch.zeros(3, dtype=torch.int32, device="cuda")
    kc = torch.ones((10, 2, 64), dtype=torch.bfloat16, device="cuda")
    hoff = torch.tensor([0, 4, 10], dtype=torch.int32, device="cuda")
    out = hstu.hstu_attn_fwd_cached(z, z, z, coff, kc, kc.clone(), hoff, 0.125, 1.0)
    assert out.shape == (0, 2, 64)
    cc = workloads.make_cached_case([0, 0], [3, 40], 2, 64, "bf16", seed=641, n=2.0)
    got = from_torch(run_cached(cc), "bf16")
    assert_close(got, oracle_cached(cc), "bf16", "cached, empty cache tensors")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_cached_null_cache_ignores_history_offsets(dtype):
    """Empty cache tensors (null cache pointers at the C ABI) with history
    offsets that claim rows: no cache row is read and every candidate sees
    itself only, as with all-zero history offsets."""
    cc = workloads.make_cached_case([0, 0, 0], [5, 70, 33], 2, 64, dtype, seed=651, n=7.0)
    q, k, v, coff, _, _, _ = device(cc)
    empty = torch.zeros((0, 2, 64), dtype=q.dtype, device="cuda")
    hoff = torch.tensor([0, 40, 40, 300], dtype=torch.int32, device="cuda")
    got = from_torch(hstu.hstu_attn_fwd_cached(q, k, v, coff, empty, empty, hoff, cc.cand.alpha,
                                               cc.cand.n), dtype)
    torch.cuda.synchronize()
    assert_close(got, oracle_cached(cc), dtype, "cached, null cache with non-zero offsets")
