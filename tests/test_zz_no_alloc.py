"""The allocation-free forward entry point (hstu_attn_fwd_noalloc, for callers
that cannot allocate) against the allocating one, hstu_attn_fwd, through the
C ABI: two calls in a row on the fixed per-GPU array, the second on a smaller
batch, each bit for bit equal to hstu_attn_fwd on the same inputs; both
table forms (one kernel up to 256 sequences, the work-list kernel above);
bf16, fp16 and fp32; a batch whose work list does not fit is refused before
anything runs.
"""
import numpy as np
import pytest

import workloads
from helpers import device_case, log

torch = pytest.importorskip("torch")
hstu = pytest.importorskip("generative_recommendation_attention_amd")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


def both(case):
    q, k, v, off = device_case(case)
    ref = hstu.hstu_attn_fwd(q, k, v, off, case.alpha, case.n)
    got = hstu.hstu_attn_fwd_noalloc(q, k, v, off, case.alpha, case.n)
    torch.cuda.synchronize()
    return ref, got


def same_bits(a, b):
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("fp16", 128), ("fp32", 64)])
def test_noalloc_two_calls_second_smaller(dtype, d):
    big = workloads.make_case([700, 1, 129, 0, 1000, 64, 257], 3, d, dtype, seed=71, n=1000.0,
                              sigma=0.5 if dtype == "fp16" else 1.0)
    small = workloads.make_case([33, 5, 200], 2, d, dtype, seed=72, n=200.0,
                                sigma=0.5 if dtype == "fp16" else 1.0)
    for what, case in (("first, larger", big), ("second, smaller", small)):
        log(f"noalloc {dtype} d={d}: {what} batch, T={case.total}")
        ref, got = both(case)
        assert same_bits(ref, got), what


def test_noalloc_two_kernel_form_then_one_kernel_form():
    """Above 256 sequences the work-list kernel builds the tables in the
    array (and zeroes its counters); the next, small call runs one kernel
    after zeroing them itself."""
    rng = np.random.default_rng(73)
    lengths = [int(x) for x in rng.integers(0, 300, size=600)]
    big = workloads.make_case(lengths, 2, 64, "bf16", seed=74, n=300.0)
    small = workloads.make_case([90, 17], 4, 64, "bf16", seed=75, n=90.0)
    for what, case in (("600 sequences", big), ("2 sequences", small), ("600 again", big)):
        log(f"noalloc: {what}, T={case.total}")
        ref, got = both(case)
        assert same_bits(ref, got), what


def test_noalloc_rejects_batch_past_the_array():
    num_seqs, heads = 20000, 16
    case = workloads.make_case([1] * num_seqs, heads, 64, "bf16", seed=76, n=1.0)
    q, k, v, off = device_case(case)
    out = torch.empty_like(q)
    with pytest.raises(hstu.HstuError) as ei:
        hstu.hstu_attn_fwd_noalloc(q, k, v, off, case.alpha, case.n, out=out)
    assert ei.value.status == hstu.HSTU_ERR_SCRATCH_LIMIT
    # the allocating entry point takes the same batch
    ref = hstu.hstu_attn_fwd(q, k, v, off, case.alpha, case.n)
    torch.cuda.synchronize()
    assert torch.isfinite(ref.float()).all().item()
