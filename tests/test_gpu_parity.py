"""Parity of the HIP path against the fp64 CPU oracle, through the C ABI.

Small cases and the five named workloads at full size (the Ascend HSTU blog's
QKV (16, 4, 4096, 64) shape of §3.2 among them, lengths up to its 20480 bound
of §3.1) are compared element by element over the whole output, with both
tolerances taken over every T * heads * d element; properties that hold at
any size (the sign-flip identity, determinism, sequence independence) are
checked as well.
"""
import numpy as np
import pytest

import oracle
import workloads
from helpers import assert_close, device_case, errors, from_torch, log, to_torch, TOL

torch = pytest.importorskip("torch")
hstu = pytest.importorskip("generative_recommendation_attention_amd")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

EDGE_LENGTHS = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 383, 0, 511, 3]


def run_gpu(case, out=None):
    q, k, v, off = device_case(case)
    res = hstu.hstu_attn_fwd(q, k, v, off, case.alpha, case.n, out=out)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
def test_edge_lengths_full_compare(dtype, d):
    heads = 2
    case = workloads.make_case(EDGE_LENGTHS, heads, d, dtype, seed=200 + d,
                               sigma=0.5 if dtype == "fp16" else 1.0,
                               alpha=1.0 / np.sqrt(d), n=float(max(EDGE_LENGTHS)))
    log(f"edge lengths {dtype} d={d} T={case.total}")
    got = from_torch(run_gpu(case), dtype)
    ref = oracle.fwd(case.q, case.k, case.v, case.offsets, heads, d, case.alpha, case.n, dtype)
    assert_close(got, ref, dtype, f"edge {dtype} d{d}")
    # Each sequence's block also meets the bar on its own (no short sequence
    # hides behind the long ones).
    for i in range(case.num_seqs):
        a, b = int(case.offsets[i]), int(case.offsets[i + 1])
        if b > a:
            mr, l2 = errors(got[a:b], ref[a:b])
            assert mr <= TOL[dtype][0] * 2 and l2 <= TOL[dtype][1] * 2, (i, b - a, mr, l2)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_many_heads_and_sequences(dtype):
    rng = np.random.default_rng(3)
    lengths = [int(x) for x in rng.integers(0, 300, size=40)]
    case = workloads.make_case(lengths, 5, 64, dtype, seed=301, alpha=0.11, n=300.0)
    log(f"many heads {dtype} T={case.total}")
    got = from_torch(run_gpu(case), dtype)
    ref = oracle.fwd(case.q, case.k, case.v, case.offsets, 5, 64, case.alpha, case.n, dtype)
    assert_close(got, ref, dtype, f"many-heads {dtype}")


def test_workload1_full_compare():
    case = workloads.workload(1)
    log("workload 1 (fp32, 1 x 256, heads 2, d 64)")
    got = from_torch(run_gpu(case), "fp32")
    ref = oracle.fwd(case.q, case.k, case.v, case.offsets, case.heads, case.d, case.alpha,
                     case.n, "fp32")
    assert_close(got, ref, "fp32", "workload 1")


@pytest.mark.parametrize("num", [2, 3, 4, 5])
def test_workload_full_compare(num):
    """The whole output of the workload against the oracle's whole output,
    in the launch configuration the benchmark times."""
    case = workloads.workload(num)
    log(f"workload {num}: {case.description}; T={case.total}")
    got = from_torch(run_gpu(case), case.dtype)
    log(f"  oracle over all {case.total * case.heads} rows")
    ref = oracle.fwd(case.q, case.k, case.v, case.offsets, case.heads, case.d, case.alpha,
                     case.n, case.dtype)
    mr, l2 = assert_close(got, ref, case.dtype, f"workload {num} whole output")
    log(f"  max|err|/max|ref| = {mr:.3e}, rel L2 = {l2:.3e} over {got.size} elements")


@pytest.mark.parametrize("num", [2, 3, 4, 5])
def test_sign_flip_identity_full_size(num):
    """hstu(Q) - hstu(-Q) = (alpha/n) tril(Q K^T) V for every sequence and head,
    checked over the whole output with torch's float32 matmul as reference."""
    case = workloads.workload(num)
    log(f"sign flip, workload {num}")
    q, k, v, off = device_case(case)
    a = hstu.hstu_attn_fwd(q, k, v, off, case.alpha, case.n).float()
    b = hstu.hstu_attn_fwd(-q, k, v, off, case.alpha, case.n).float()
    diff = a - b
    num_err = 0.0
    den = 0.0
    offs = case.offsets
    qf, kf, vf = q.float(), k.float(), v.float()
    for i in range(case.num_seqs):
        s0, s1 = int(offs[i]), int(offs[i + 1])
        if s1 == s0:
            continue
        Q = qf[s0:s1].transpose(0, 1).contiguous()  # (H, s, d)
        K = kf[s0:s1].transpose(0, 1).contiguous()
        V = vf[s0:s1].transpose(0, 1).contiguous()
        S = torch.tril(torch.matmul(Q, K.transpose(1, 2).contiguous()))
        R = (case.alpha / case.n) * torch.matmul(S, V)
        D = diff[s0:s1].transpose(0, 1)
        num_err += float(((D - R) ** 2).sum())
        den += float((R ** 2).sum())
    rel = (num_err / den) ** 0.5
    log(f"  rel L2 = {rel:.3e}")
    assert rel <= 1e-2


def test_deterministic_and_sequence_independent():
    case = workloads.make_case([700, 1, 129, 0, 1000, 64], 3, 128, "bf16", seed=9, n=1000.0)
    q, k, v, off = device_case(case)
    a = hstu.hstu_attn_fwd(q, k, v, off, case.alpha, case.n)
    b = hstu.hstu_attn_fwd(q, k, v, off, case.alpha, case.n)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # One call per sequence gives the same bits as the batched call.
    for i in range(case.num_seqs):
        s0, s1 = int(case.offsets[i]), int(case.offsets[i + 1])
        if s1 == s0:
            continue
        one = hstu.hstu_attn_fwd(q[s0:s1].contiguous(), k[s0:s1].contiguous(),
                                 v[s0:s1].contiguous(),
                                 torch.tensor([0, s1 - s0], dtype=torch.int32, device="cuda"),
                                 case.alpha, case.n)
        assert torch.equal(one.view(torch.int16), a[s0:s1].view(torch.int16)), i


def test_guard_bands_untouched():
    """out placed inside a larger buffer filled with NaN: only its own rows change."""
    case = workloads.make_case([300, 17, 0, 129], 2, 64, "bf16", seed=12, n=300.0)
    q, k, v, off = device_case(case)
    T, H, D = case.total, case.heads, case.d
    pad = 4096
    buf = torch.full((pad + T * H * D + pad,), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = buf[pad:pad + T * H * D].view(T, H, D)
    hstu.hstu_attn_fwd(q, k, v, off, case.alpha, case.n, out=out)
    torch.cuda.synchronize()
    assert torch.isnan(buf[:pad].float()).all() and torch.isnan(buf[-pad:].float()).all()
    ref = oracle.fwd(case.q, case.k, case.v, case.offsets, H, D, case.alpha, case.n, "bf16")
    assert_close(from_torch(out, "bf16"), ref, "bf16", "guard-band case")


def test_inputs_in_guarded_buffers():
    """q/k/v as views inside NaN-filled buffers: no read past the last token."""
    case = workloads.make_case([65, 200, 3], 2, 128, "fp16", seed=13, sigma=0.5, n=200.0)
    T, H, D = case.total, case.heads, case.d
    pad = 8 * H * D
    views = []
    for x in (case.q, case.k, case.v):
        buf = torch.full((pad + T * H * D + pad,), float("nan"), dtype=torch.float16,
                         device="cuda")
        view = buf[pad:pad + T * H * D].view(T, H, D)
        view.copy_(to_torch(x, "fp16"))
        views.append(view)
    off = torch.from_numpy(case.offsets).cuda()
    got = hstu.hstu_attn_fwd(*views, off, case.alpha, case.n)
    ref = oracle.fwd(case.q, case.k, case.v, case.offsets, H, D, case.alpha, case.n, "fp16")
    assert_close(from_torch(got, "fp16"), ref, "fp16", "guarded inputs")


def test_empty_batch_and_zero_length_only():
    q = torch.zeros((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    off = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = hstu.hstu_attn_fwd(q, q, q, off, 0.125, 1.0)
    assert out.shape == (0, 2, 64)
    # Four sequences, all empty: nothing to compute, nothing written.
    x = torch.zeros((1, 2, 64), dtype=torch.bfloat16, device="cuda")
    off = torch.zeros(5, dtype=torch.int32, device="cuda")
    out = torch.full_like(x, 7.0)
    hstu.hstu_attn_fwd(x, x.clone(), x.clone(), off, 0.125, 1.0, out=out)
    torch.cuda.synchronize()
    assert (out.float() == 7.0).all()


def test_validate_offsets():
    good = torch.tensor([0, 3, 3, 10], dtype=torch.int32, device="cuda")
    assert hstu.hstu_validate_offsets(good) == 10
    bad = torch.tensor([0, 5, 4], dtype=torch.int32, device="cuda")
    with pytest.raises(hstu.HstuError):
        hstu.hstu_validate_offsets(bad)


def test_more_sequences_than_the_sort_takes():
    """Above the one-workgroup sort's limit the work list falls back to input
    order; results must not change."""
    rng = np.random.default_rng(17)
    lengths = [int(x) for x in rng.integers(0, 40, size=20000)]
    case = workloads.make_case(lengths, 1, 64, "bf16", seed=18, n=40.0)
    log(f"20000 sequences, T={case.total}")
    got = from_torch(run_gpu(case), "bf16")
    ref = oracle.fwd(case.q, case.k, case.v, case.offsets, 1, 64, case.alpha, case.n, "bf16")
    assert_close(got, ref, "bf16", "20000 sequences")


@pytest.mark.parametrize("sort", ["bitonic", "input"])
def test_scheduler_ranking_paths_agree(sort, monkeypatch):
    """Every ranking path of the scheduler (counting sort, bitonic sort, input
    order) must give bit-identical output: an item's result never depends on
    which workgroup runs it or when."""
    rng = np.random.default_rng(23)
    lengths = [int(x) for x in rng.integers(0, 700, size=300)]
    case = workloads.make_case(lengths, 2, 64, "bf16", seed=24, n=700.0)
    q, k, v, off = device_case(case)
    ref = hstu.hstu_attn_fwd(q, k, v, off, case.alpha, case.n)
    monkeypatch.setenv("HSTU_SCHED_SORT", sort)
    got = hstu.hstu_attn_fwd(q, k, v, off, case.alpha, case.n)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_profiling_counts_calls():
    # A small batch runs as one kernel (no work-list kernel time); a batch of
    # more than 256 sequences runs the work-list kernel first.
    for lengths, one_kernel in (([512, 512], True), ([40] * 300, False)):
        case = workloads.make_case(lengths, 2, 64, "bf16", seed=19, n=512.0)
        q, k, v, off = device_case(case)
        hstu.hstu_attn_fwd(q, k, v, off, case.alpha, case.n)   # scratch sized outside the count
        hstu.hstu_profile_read(reset=True)
        hstu.hstu_profile_enable(True)
        for _ in range(3):
            hstu.hstu_attn_fwd(q, k, v, off, case.alpha, case.n)
        hstu.hstu_profile_enable(False)
        t = hstu.hstu_profile_read(reset=True)
        assert t.calls == 3 and t.attn_ms > 0
        assert (t.sched_ms == 0) if one_kernel else (t.sched_ms > 0)
