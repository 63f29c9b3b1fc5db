"""Edge cases of the forward against the fp64 oracle: the longest sequence the
pages use (20480 tokens, the Ascend HSTU blog's length bound), many heads,
alpha = 0 (every weight silu(0) = 0), scores large enough that SiLU saturates
on both sides, a one-token batch, and very small / large n.
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


def run(case):
    q, k, v, off = device_case(case)
    out = hstu.hstu_attn_fwd(q, k, v, off, case.alpha, case.n)
    torch.cuda.synchronize()
    return out


def test_longest_sequence_full_compare():
    case = workloads.make_case([20480], 4, 64, "bf16", seed=950, alpha=0.125, n=20480.0)
    log("one sequence of 20480 tokens, heads 4, d 64, bf16")
    got = from_torch(run(case), "bf16")
    ref = oracle.fwd(case.q, case.k, case.v, case.offsets, 4, 64, case.alpha, case.n, "bf16")
    mr, l2 = assert_close(got, ref, "bf16", "20480-token sequence")
    log(f"  max|err|/max|ref| = {mr:.3e}, rel L2 = {l2:.3e}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_sixteen_heads_d128(dtype):
    case = workloads.make_case([300, 17, 129], 16, 128, dtype, seed=951,
                               sigma=0.5 if dtype == "fp16" else 1.0, n=300.0)
    got = from_torch(run(case), dtype)
    ref = oracle.fwd(case.q, case.k, case.v, case.offsets, 16, 128, case.alpha, case.n, dtype)
    assert_close(got, ref, dtype, f"16 heads d128 {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_alpha_zero_gives_zero(dtype):
    case = workloads.make_case([100, 300], 2, 64, dtype, seed=952, alpha=0.0, n=3.0)
    out = run(case)
    assert torch.count_nonzero(out.float()).item() == 0


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_saturating_scores(dtype):
    """alpha = 4 with unit-variance q, k of d = 64: scores of magnitude in the
    hundreds, where silu(x) is x on one side and 0 on the other."""
    case = workloads.make_case([257, 64], 2, 64, dtype, seed=953, alpha=4.0, n=257.0)
    got = from_torch(run(case), dtype)
    assert np.all(np.isfinite(got))
    ref = oracle.fwd(case.q, case.k, case.v, case.offsets, 2, 64, case.alpha, case.n, dtype)
    assert_close(got, ref, dtype, f"saturating {dtype}")


@pytest.mark.parametrize("n", [1e-3, 1.0, 1e6])
def test_normaliser_extremes(n):
    case = workloads.make_case([70, 200], 2, 128, "bf16", seed=954, n=n)
    got = from_torch(run(case), "bf16")
    ref = oracle.fwd(case.q, case.k, case.v, case.offsets, 2, 128, case.alpha, case.n, "bf16")
    assert_close(got, ref, "bf16", f"n = {n}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_single_token_batch(dtype):
    case = workloads.make_case([1], 1, 64, dtype, seed=955, n=1.0)
    got = from_torch(run(case), dtype)
    ref = oracle.fwd(case.q, case.k, case.v, case.offsets, 1, 64, case.alpha, case.n, dtype)
    assert_close(got, ref, dtype, f"one token {dtype}")
