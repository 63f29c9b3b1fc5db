"""Parity of the backward (dq, dk, dv) against the fp64 CPU oracle, through
the C ABI.

The tolerance is the forward's (bf16/fp16: max|err| <= 1e-2 max|ref|, rel L2
<= 5e-3; fp32 1e-4 on both): an emulation of the kernels' roundings (P and the score gradient
rounded to bf16 before their products, fp32 accumulation, outputs rounded)
gives about 2.4e-3 relative L2 and 2-4e-3 max ratio at 256-1024 tokens.
Small cases and workloads 2 and 3 are compared element by element.
"""
import numpy as np
import pytest

import oracle
import workloads
from helpers import TOL, assert_close, device_case, errors, from_torch, log, to_torch

torch = pytest.importorskip("torch")
hstu = pytest.importorskip("generative_recommendation_attention_amd")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

EDGE_LENGTHS = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 383, 0, 511, 3]


def with_dout(case, seed):
    """An upstream gradient drawn like q (its own seed)."""
    return workloads.make_case(list(case.lengths), case.heads, case.d, case.dtype, seed=seed,
                               sigma=0.5 if case.dtype == "fp16" else 1.0).q


def run_bwd(case, dout, num_targets=None):
    q, k, v, off = device_case(case)
    do = to_torch(dout, case.dtype)
    tg = None if num_targets is None else torch.tensor(num_targets, dtype=torch.int32).cuda()
    res = hstu.hstu_attn_bwd(q, k, v, do, off, case.alpha, case.n, num_targets=tg)
    torch.cuda.synchronize()
    return [from_torch(x, case.dtype) for x in res]


def check_all(got, ref, dtype, what, per_seq_offsets=None):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert_close(g, r, dtype, f"{what} {name}")
        if per_seq_offsets is not None:
            off = per_seq_offsets
            for i in range(len(off) - 1):
                a, b = int(off[i]), int(off[i + 1])
                if b > a and np.max(np.abs(r[a:b])) > 0:
                    mr, l2 = errors(g[a:b], r[a:b])
                    assert mr <= TOL[dtype][0] * 2 and l2 <= TOL[dtype][1] * 2, \
                        (what, name, i, b - a, mr, l2)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
def test_bwd_edge_lengths_full_compare(dtype, d):
    case = workloads.make_case(EDGE_LENGTHS, 2, d, dtype, seed=700 + d,
                               sigma=0.5 if dtype == "fp16" else 1.0, alpha=1.0 / np.sqrt(d),
                               n=511.0)
    dout = with_dout(case, 710 + d)
    log(f"bwd edge {dtype} d={d} T={case.total}")
    got = run_bwd(case, dout)
    ref = oracle.bwd(case.q, case.k, case.v, dout, case.offsets, 2, d, case.alpha, case.n, dtype)
    check_all(got, ref, dtype, f"bwd edge {dtype} d{d}", case.offsets)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
def test_bwd_targets_full_compare(dtype, d):
    pairs = [(1, 1), (2, 5), (31, 0), (32, 1), (33, 2), (63, 31), (64, 32), (65, 33),
             (127, 64), (128, 100), (129, 128), (255, 200), (256, 255), (257, 1), (383, 350),
             (0, 0), (511, 17), (3, -4), (300, 64), (200, 200), (450, 97), (97, 96)]
    case = workloads.make_case([s for s, _ in pairs], 2, d, dtype, seed=720 + d,
                               sigma=0.5 if dtype == "fp16" else 1.0, alpha=1.0 / np.sqrt(d),
                               n=511.0)
    tg = [t for _, t in pairs]
    dout = with_dout(case, 730 + d)
    log(f"bwd targets {dtype} d={d} T={case.total}")
    got = run_bwd(case, dout, tg)
    ref = oracle.bwd(case.q, case.k, case.v, dout, case.offsets, 2, d, case.alpha, case.n, dtype,
                     num_targets=tg)
    check_all(got, ref, dtype, f"bwd targets {dtype} d{d}", case.offsets)


def test_bwd_many_sequences_two_kernel_form():
    rng = np.random.default_rng(37)
    lengths = rng.integers(0, 260, size=300).tolist()
    case = workloads.make_case(lengths, 3, 64, "bf16", seed=741, alpha=0.1, n=260.0)
    dout = with_dout(case, 742)
    log(f"bwd 300 sequences T={case.total}")
    got = run_bwd(case, dout)
    ref = oracle.bwd(case.q, case.k, case.v, dout, case.offsets, 3, 64, case.alpha, case.n,
                     "bf16")
    check_all(got, ref, "bf16", "bwd 300 sequences")


def test_bwd_value_identity_full_size():
    """out is linear in v, so <dv, v> = <dout, out>: GPU backward against GPU
    forward at 16 x 4096 (relative 1e-2)."""
    case = workloads.workload(2)
    dout = with_dout(case, 751)
    q, k, v, off = device_case(case)
    do = to_torch(dout, "bf16")
    out = hstu.hstu_attn_fwd(q, k, v, off, case.alpha, case.n).float()
    dq, dk, dv = hstu.hstu_attn_bwd(q, k, v, do, off, case.alpha, case.n)
    lhs = float((dv.float() * v.float()).sum())
    rhs = float((do.float() * out).sum())
    log(f"  <dv, v> = {lhs:.6e}, <dout, out> = {rhs:.6e}")
    assert abs(lhs - rhs) <= 1e-2 * abs(rhs)
    for x in (dq, dk, dv):
        assert torch.isfinite(x.float()).all().item()


@pytest.mark.parametrize("num", [2, 3])
def test_bwd_workload_full_compare(num):
    """Workload 2 (16 x 4096, heads 4, d 64, the forward's headline shape) and
    workload 3 (64 skewed sequences up to 8192, heads 4, d 128), bf16: every
    element of dq, dk and dv against the fp64 oracle (about 30 s and 2 min of
    oracle time on 16 host threads)."""
    case = workloads.workload(num)
    dout = with_dout(case, 760 + num)
    log(f"bwd workload {num} whole output: {case.description}")
    got = run_bwd(case, dout)
    ref = oracle.bwd(case.q, case.k, case.v, dout, case.offsets, case.heads, case.d,
                     case.alpha, case.n, case.dtype)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        mr, l2 = assert_close(g, r, case.dtype, f"bwd workload {num} {name}")
        log(f"  {name}: max|err|/max|ref| = {mr:.3e}, rel L2 = {l2:.3e}")


def test_bwd_fp32_many_sequences_two_kernel_form():
    rng = np.random.default_rng(38)
    lengths = rng.integers(0, 200, size=290).tolist()
    case = workloads.make_case(lengths, 2, 128, "fp32", seed=771, alpha=0.1, n=200.0)
    dout = with_dout(case, 772)
    got = run_bwd(case, dout)
    ref = oracle.bwd(case.q, case.k, case.v, dout, case.offsets, 2, 128, case.alpha, case.n,
                     "fp32")
    check_all(got, ref, "fp32", "bwd fp32 290 sequences")
