"""The dense (batch, heads, seq_len, d) forward (the Ascend HSTU blog's §1
layout) against the fp64 oracle, through the C ABI.

The oracle takes the jagged (T, heads, d) layout; the test re-lays the dense
inputs on the host (a transpose, no arithmetic).  The dense call must also
agree bit for bit with the jagged call on the re-laid inputs (the kernels do
the same arithmetic in the same order; only the addressing differs).
"""
import numpy as np
import pytest

import oracle
import workloads
from helpers import assert_close, from_torch, log, to_torch

torch = pytest.importorskip("torch")
hstu = pytest.importorskip("generative_recommendation_attention_amd")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


def dense_case(B, H, S, d, dtype, seed, alpha=None, n=None):
    """A jagged case of B equal sequences plus its dense (B, H, S, d) image."""
    case = workloads.make_case([S] * B, H, d, dtype, seed=seed,
                               sigma=0.5 if dtype == "fp16" else 1.0, alpha=alpha,
                               n=n if n is not None else float(max(S, 1)))
    dense = [np.ascontiguousarray(x.reshape(B, S, H, d).transpose(0, 2, 1, 3))
             for x in (case.q, case.k, case.v)]
    return case, dense


def to_jagged(x, B, H, S, d):
    return np.ascontiguousarray(x.reshape(B, H, S, d).transpose(0, 2, 1, 3)).reshape(B * S, H, d)


def run_dense(case, dense, B, H, S, d):
    q, k, v = (to_torch(x, case.dtype) for x in dense)
    out = hstu.hstu_attn_fwd_dense(q, k, v, case.alpha, case.n)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("S", [1, 33, 257])
def test_dense_full_compare(dtype, d, S):
    B, H = 3, 2
    case, dense = dense_case(B, H, S, d, dtype, seed=800 + S + d)
    log(f"dense {dtype} d={d} B={B} H={H} S={S}")
    out = run_dense(case, dense, B, H, S, d)
    got = to_jagged(from_torch(out, dtype), B, H, S, d)
    ref = oracle.fwd(case.q, case.k, case.v, case.offsets, H, d, case.alpha, case.n, dtype)
    assert_close(got, ref, dtype, f"dense {dtype} d{d} S{S}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_dense_matches_jagged_bitwise(dtype):
    B, H, S, d = 5, 3, 300, 64
    case, dense = dense_case(B, H, S, d, dtype, seed=811)
    a = run_dense(case, dense, B, H, S, d)
    q, k, v = (to_torch(x, dtype) for x in (case.q, case.k, case.v))
    off = torch.from_numpy(case.offsets).cuda()
    b = hstu.hstu_attn_fwd(q, k, v, off, case.alpha, case.n)
    torch.cuda.synchronize()
    dj = torch.from_numpy(to_jagged(from_torch(a, dtype), B, H, S, d))
    assert torch.equal(dj, torch.from_numpy(from_torch(b, dtype)))


def test_dense_offset_ramp_reuse_and_invalidation():
    """Dense calls of different shapes, with a jagged call of many sequences
    between them (its work list overwrites the stored offsets), each checked."""
    shapes = [(2, 2, 100), (7, 1, 40), (2, 2, 100)]
    for i, (B, H, S) in enumerate(shapes):
        case, dense = dense_case(B, H, S, 64, "bf16", seed=820 + i)
        got = to_jagged(from_torch(run_dense(case, dense, B, H, S, 64), "bf16"), B, H, S, 64)
        ref = oracle.fwd(case.q, case.k, case.v, case.offsets, H, 64, case.alpha, case.n, "bf16")
        assert_close(got, ref, "bf16", f"dense {B}x{H}x{S}")
        many = workloads.make_case([3] * 600, 2, 64, "bf16", seed=830 + i)
        q, k, v = (to_torch(x, "bf16") for x in (many.q, many.k, many.v))
        hstu.hstu_attn_fwd(q, k, v, torch.from_numpy(many.offsets).cuda(), many.alpha, many.n)
    torch.cuda.synchronize()


def test_dense_blog_shape_whole_output_and_sampled_rows():
    """QKV (16, 4, 4096, 64) in bf16, the shape the blog times: the whole
    output, and sampled rows through the oracle's row function."""
    B, H, S, d = 16, 4, 4096, 64
    case, dense = dense_case(B, H, S, d, "bf16", seed=840, alpha=0.125, n=4096.0)
    out = run_dense(case, dense, B, H, S, d)
    rng = np.random.default_rng(5)
    bs = rng.integers(0, B, size=40)
    hs = rng.integers(0, H, size=40)
    rs = np.concatenate([[0, 63, 64, 255, 256, 4095], rng.integers(0, S, size=34)])
    got = from_torch(out[torch.from_numpy(bs).cuda(), torch.from_numpy(hs).cuda(),
                         torch.from_numpy(rs).cuda()], "bf16")
    tok = (bs * S + rs).astype(np.int64)
    ref = oracle.rows(case.q, case.k, case.v, case.offsets, H, d, case.alpha, case.n, "bf16",
                      tok, hs.astype(np.int32))
    mr, l2 = assert_close(got, ref, "bf16", "dense blog shape")
    log(f"  max|err|/max|ref| = {mr:.3e}, rel L2 = {l2:.3e}")
    whole = to_jagged(from_torch(out, "bf16"), B, H, S, d)
    ref = oracle.fwd(case.q, case.k, case.v, case.offsets, H, d, case.alpha, case.n, "bf16")
    mr, l2 = assert_close(whole, ref, "bf16", "dense blog shape whole output")
    log(f"  whole output: max|err|/max|ref| = {mr:.3e}, rel L2 = {l2:.3e}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
def test_dense_backward_full_compare(dtype, d):
    B, H, S = 3, 2, 200
    case, dense = dense_case(B, H, S, d, dtype, seed=850 + d)
    dout_j = workloads.make_case([S] * B, H, d, dtype, seed=851,
                                 sigma=0.5 if dtype == "fp16" else 1.0).q
    dout = np.ascontiguousarray(dout_j.reshape(B, S, H, d).transpose(0, 2, 1, 3))
    q, k, v, do = (to_torch(x, dtype) for x in (*dense, dout))
    grads = hstu.hstu_attn_bwd_dense(q, k, v, do, case.alpha, case.n)
    torch.cuda.synchronize()
    ref = oracle.bwd(case.q, case.k, case.v, dout_j, case.offsets, H, d, case.alpha, case.n,
                     dtype)
    for name, g, r in zip(("dq", "dk", "dv"), grads, ref):
        got = to_jagged(from_torch(g, dtype), B, H, S, d)
        assert_close(got, r, dtype, f"dense backward {name} {dtype} d{d}")
