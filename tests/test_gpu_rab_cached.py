"""Parity of the cached-history forward with the relative attention bias
against the fp64 CPU oracle, through the C ABI (HSTU paper translation §3.4:
M-FALCON adjusts rab_{p,t} with the mask; Appendix H: the history's K and V
come from a cache).  The oracle's reading: a candidate sits right after its
request's cached history (distance h - c to cached row c, 0 to itself) and
keeps its own timestamp; the history rows keep theirs.

Small cases are compared element by element: histories on and around the
32/64-key tiles (the kernel pads the history to whole tiles and reads zero K,
V and timestamps there), empty histories and micro-batches, position tables
shorter than the distances.  The 16 x (3072 cached + 1024 candidates)
workload element by element and on sampled rows.  Properties: zero tables give the cached forward
without bias bit for bit; the result equals the candidate rows of one
target-aware bias pass over history + candidates (GPU against GPU, within the
tolerance: the candidates' own keys sit in other key blocks there).
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

# (history rows, candidates): empty history, empty micro-batch, histories on
# and around key-tile edges (32 and 64 keys), candidates across query tiles.
EDGE = [(0, 5), (1, 1), (31, 2), (32, 33), (33, 64), (63, 1), (64, 100), (65, 128),
        (100, 0), (127, 129), (128, 255), (129, 256), (300, 257), (511, 31), (0, 0),
        (2, 300), (97, 3), (256, 1), (700, 40)]


def make(hist, cand, heads, d, dtype, seed, npos, ntime, sigma=1.0, alpha=None, n=None):
    cc = workloads.make_cached_case(hist, cand, heads, d, dtype, seed=seed, sigma=sigma,
                                    alpha=alpha, n=n)
    r, hts = workloads.make_cached_rab_inputs(cc.hist_offsets, cc.cand.offsets, npos, ntime,
                                              seed=seed + 1)
    return cc, r, hts


def device(cc):
    c = cc.cand
    dt = c.dtype
    return (to_torch(c.q, dt), to_torch(c.k, dt), to_torch(c.v, dt),
            torch.from_numpy(c.offsets.astype(np.int32)).cuda(),
            to_torch(cc.k_cache, dt), to_torch(cc.v_cache, dt),
            torch.from_numpy(cc.hist_offsets.astype(np.int32)).cuda())


def run(cc, r, hts):
    q, k, v, coff, kc, vc, hoff = device(cc)
    res = hstu.hstu_attn_fwd_rab_cached(q, k, v, coff, kc, vc, hoff,
                                        torch.from_numpy(r.timestamps).cuda(),
                                        torch.from_numpy(hts).cuda(),
                                        torch.from_numpy(r.pos_bias).cuda(),
                                        torch.from_numpy(r.time_bias).cuda(), cc.cand.alpha,
                                        cc.cand.n)
    torch.cuda.synchronize()
    return res


def oracle_fwd(cc, r, hts):
    c = cc.cand
    return oracle.fwd_rab_cached(c.q, c.k, c.v, c.offsets, cc.k_cache, cc.v_cache,
                                 cc.hist_offsets, r.timestamps, hts, r.pos_bias, r.time_bias,
                                 c.heads, c.d, c.alpha, c.n, c.dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("npos,ntime", [(800, 16), (40, 32)])
def test_rab_cached_edge_full_compare(dtype, d, npos, ntime):
    cc, r, hts = make([h for h, _ in EDGE], [t for _, t in EDGE], 2, d, dtype,
                      seed=1700 + d + npos, npos=npos, ntime=ntime,
                      sigma=0.5 if dtype == "fp16" else 1.0, alpha=1.0 / np.sqrt(d), n=811.0)
    log(f"rab cached edge {dtype} d={d} npos={npos} Tc={cc.cand.total} "
        f"Th={int(cc.hist_offsets[-1])}")
    got = from_torch(run(cc, r, hts), dtype)
    ref = oracle_fwd(cc, r, hts)
    assert_close(got, ref, dtype, f"rab cached edge {dtype} d{d}")
    off = cc.cand.offsets
    for i in range(cc.cand.num_seqs):
        a, b = int(off[i]), int(off[i + 1])
        if b > a:
            mr, l2 = errors(got[a:b], ref[a:b])
            assert mr <= TOL[dtype][0] * 2 and l2 <= TOL[dtype][1] * 2, (i, EDGE[i], mr, l2)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("fp16", 128), ("fp32", 64)])
def test_zero_tables_match_cached_without_bias_bitwise(dtype, d):
    cc, r, hts = make([h for h, _ in EDGE], [t for _, t in EDGE], 2, d, dtype, seed=1730,
                      npos=50, ntime=6, sigma=0.5 if dtype == "fp16" else 1.0)
    r.pos_bias[:] = 0
    r.time_bias[:] = 0
    got = run(cc, r, hts)
    q, k, v, coff, kc, vc, hoff = device(cc)
    plain = hstu.hstu_attn_fwd_cached(q, k, v, coff, kc, vc, hoff, cc.cand.alpha, cc.cand.n)
    torch.cuda.synchronize()
    view = torch.int32 if dtype == "fp32" else torch.int16
    assert torch.equal(got.view(view), plain.view(view))


def test_rab_cached_equals_one_target_aware_bias_pass():
    """The candidates get what one target-aware bias pass over history +
    candidates gives them (both on the GPU; timestamps and tables shared)."""
    hist, cand = [700, 64, 0, 129, 1], [45, 200, 7, 64, 3]
    cc, r, hts = make(hist, cand, 2, 64, "bf16", seed=1740, npos=900, ntime=12,
                      alpha=0.125, n=900.0)
    got = from_torch(run(cc, r, hts), "bf16")
    c = cc.cand
    qs, ks, vs, ts, lens = [], [], [], [], []
    for i in range(c.num_seqs):
        ha, hb = int(cc.hist_offsets[i]), int(cc.hist_offsets[i + 1])
        ca, cb = int(c.offsets[i]), int(c.offsets[i + 1])
        qs += [np.zeros_like(cc.k_cache[ha:hb]), c.q[ca:cb]]
        ks += [cc.k_cache[ha:hb], c.k[ca:cb]]
        vs += [cc.v_cache[ha:hb], c.v[ca:cb]]
        ts += [hts[ha:hb], r.timestamps[ca:cb]]
        lens.append(hb - ha + cb - ca)
    off = workloads.offsets_from_lengths(lens)
    q, k, v = (to_torch(np.concatenate(x), "bf16") for x in (qs, ks, vs))
    full = hstu.hstu_attn_fwd_rab_targets(q, k, v, torch.from_numpy(off).cuda(),
                                          torch.tensor(cand, dtype=torch.int32).cuda(),
                                          torch.from_numpy(np.concatenate(ts)).cuda(),
                                          torch.from_numpy(r.pos_bias).cuda(),
                                          torch.from_numpy(r.time_bias).cuda(), c.alpha, c.n)
    full = from_torch(full, "bf16")
    ref = np.concatenate([full[int(off[i]) + hist[i]:int(off[i + 1])] for i in range(len(hist))])
    mr, l2 = errors(got, ref)
    log(f"  rab cached vs one target-aware pass: {mr:.3e} {l2:.3e}")
    assert mr <= TOL["bf16"][0] and l2 <= TOL["bf16"][1]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_rab_cached_many_requests_two_kernel_form(dtype):
    """More requests than the one-kernel form takes: the work-list kernel runs."""
    rng = np.random.default_rng(23)
    hist = rng.integers(0, 150, size=300).tolist()
    cand = rng.integers(0, 90, size=300).tolist()
    cc, r, hts = make(hist, cand, 3, 64, dtype, seed=1750, npos=120, ntime=10, alpha=0.1,
                      n=240.0)
    log(f"rab cached 300 requests {dtype} Tc={cc.cand.total}")
    got = from_torch(run(cc, r, hts), dtype)
    assert_close(got, oracle_fwd(cc, r, hts), dtype, f"rab cached 300 requests {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_rab_cached_null_cache_ignores_history_offsets(dtype):
    """Empty cache tensors (null cache and history-timestamp pointers at the C
    ABI) with history offsets that claim rows: every candidate sees itself
    only, at distance 0 and gap 0."""
    cc, r, hts = make([0, 0, 0], [5, 70, 33], 2, 64, dtype, seed=1760, npos=30, ntime=8, n=7.0)
    q, k, v, coff, _, _, _ = device(cc)
    empty = torch.zeros((0, 2, 64), dtype=q.dtype, device="cuda")
    hoff = torch.tensor([0, 40, 40, 300], dtype=torch.int32, device="cuda")
    got = hstu.hstu_attn_fwd_rab_cached(q, k, v, coff, empty, empty, hoff,
                                        torch.from_numpy(r.timestamps).cuda(),
                                        torch.zeros(0, dtype=torch.int32, device="cuda"),
                                        torch.from_numpy(r.pos_bias).cuda(),
                                        torch.from_numpy(r.time_bias).cuda(), cc.cand.alpha,
                                        cc.cand.n)
    torch.cuda.synchronize()
    assert_close(from_torch(got, dtype), oracle_fwd(cc, r, hts), dtype,
                 "rab cached, null cache with non-zero offsets")


def test_rab_cached_workload_whole_output_and_sampled_rows():
    """16 x (3072 cached + 1024 candidates), heads 4, d 64, bf16, a position
    entry per distance and 16 time buckets: the whole output, and sampled
    candidate rows through the oracle's row function."""
    cc, r, hts = workloads.rab_cached_workload()
    c = cc.cand
    log(f"rab cached workload: Tc={c.total} Th={int(cc.hist_offsets[-1])}")
    got = run(cc, r, hts)
    rng = np.random.default_rng(17)
    rows = np.concatenate([[0, 1, 31, 32, 63, 64, 127, 128, 1023],
                           rng.integers(0, 1024, size=7)])
    seqs = rng.integers(0, 16, size=len(rows))
    tok = (seqs * 1024 + rows).astype(np.int64)
    hd = rng.integers(0, 4, size=len(tok)).astype(np.int32)
    g = from_torch(got[torch.from_numpy(tok).cuda(), torch.from_numpy(hd.astype(np.int64)).cuda()],
                   c.dtype)
    ref = oracle.rows_rab_cached(c.q, c.k, c.v, c.offsets, cc.k_cache, cc.v_cache,
                                 cc.hist_offsets, r.timestamps, hts, r.pos_bias, r.time_bias,
                                 c.heads, c.d, c.alpha, c.n, c.dtype, tok, hd)
    mr, l2 = assert_close(g, ref, c.dtype, "rab cached workload sampled")
    log(f"  max|err|/max|ref| = {mr:.3e}, rel L2 = {l2:.3e}")
    mr, l2 = assert_close(from_torch(got, c.dtype), oracle_fwd(cc, r, hts), c.dtype,
                          "rab cached workload whole output")
    log(f"  whole output: max|err|/max|ref| = {mr:.3e}, rel L2 = {l2:.3e}")
    assert torch.isfinite(got.float()).all().item()


def test_rab_cached_binding_rejects_bad_timestamps():
    cc, r, hts = make([3, 2], [2, 1], 1, 64, "bf16", seed=1, npos=8, ntime=4)
    q, k, v, coff, kc, vc, hoff = device(cc)
    ts = torch.from_numpy(r.timestamps).cuda()
    wp, wt = torch.from_numpy(r.pos_bias).cuda(), torch.from_numpy(r.time_bias).cuda()
    with pytest.raises(ValueError):   # history timestamps of the wrong length
        hstu.hstu_attn_fwd_rab_cached(q, k, v, coff, kc, vc, hoff, ts,
                                      torch.from_numpy(hts[:-1]).cuda(), wp, wt, 0.1, 1.0)
    with pytest.raises(ValueError):   # candidate timestamps of the wrong length
        hstu.hstu_attn_fwd_rab_cached(q, k, v, coff, kc, vc, hoff, ts[:-1],
                                      torch.from_numpy(hts).cuda(), wp, wt, 0.1, 1.0)
