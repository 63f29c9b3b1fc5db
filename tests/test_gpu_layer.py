"""The layer's surroundings (input projection with SiLU and split; layer norm
times U with output projection and residual) against the fp64 oracle,
through the C ABI.

Every case, up to the 65536 tokens of the 16 x 4096 workload, is compared
element by element.  Tolerance: the attention's (bf16/fp16 max|err| <=
1e-2 max|ref|, rel L2 <= 5e-3); the kernels round the normalised, gated rows
to the input type before the output product, and every output once.
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

SHAPES = [(128, 2, 64), (256, 4, 64), (512, 4, 128), (256, 2, 128), (512, 8, 64)]


def vals(shape, seed, dtype, scale=1.0):
    rng = np.random.default_rng(seed)
    return workloads.cast_values((rng.standard_normal(shape) * scale).astype(np.float32), dtype)


def params(n, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(n) * scale).astype(np.float32)


def f32dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("dm,H,d", SHAPES)
@pytest.mark.parametrize("T", [1, 127, 300])
def test_layer_in_full_compare(dtype, dm, H, d, T):
    hd = H * d
    x = vals((T, dm), 900 + T, dtype)
    w1 = vals((4 * hd, dm), 901, dtype, 1.0 / np.sqrt(dm))
    b1 = params(4 * hd, 902, 0.1)
    out = hstu.hstu_layer_in_proj(to_torch(x, dtype), to_torch(w1, dtype), f32dev(b1), H, d)
    torch.cuda.synchronize()
    ref = oracle.layer_in(x, w1, b1.astype(np.float64), H, d, dtype)
    for name, g, r in zip("uvqk", out, ref):
        assert_close(from_torch(g, dtype), r, dtype, f"layer_in {name} {dtype} {dm} {H}x{d} T{T}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("dm,H,d", SHAPES)
@pytest.mark.parametrize("T", [1, 127, 300])
def test_layer_out_full_compare(dtype, dm, H, d, T):
    hd = H * d
    attn = vals((T, H, d), 910 + T, dtype, 0.05)
    u = vals((T, H, d), 911, dtype)
    x = vals((T, dm), 912, dtype)
    w2 = vals((dm, hd), 913, dtype, 1.0 / np.sqrt(hd))
    gamma, beta, b2 = 1.0 + params(hd, 914, 0.1), params(hd, 915, 0.1), params(dm, 916, 0.1)
    eps = 1e-5
    y = hstu.hstu_layer_out_proj(to_torch(attn, dtype), to_torch(u, dtype), to_torch(x, dtype),
                                 f32dev(gamma), f32dev(beta), eps, to_torch(w2, dtype),
                                 f32dev(b2))
    torch.cuda.synchronize()
    ref = oracle.layer_out(attn, u, x, gamma.astype(np.float64), beta.astype(np.float64),
                           float(np.float32(eps)), w2, b2.astype(np.float64), H, d, dtype)
    assert_close(from_torch(y, dtype), ref, dtype, f"layer_out {dtype} {dm} {H}x{d} T{T}")


def test_layer_full_size_whole_output():
    """65536 tokens, d_model 256, heads 4, d 64 (the 16 x 4096 workload's
    projections), bf16: every element of u, v, q, k and y through the
    oracle (about 10 s of oracle time on 16 host threads)."""
    dtype, T, dm, H, d = "bf16", 65536, 256, 4, 64
    hd = H * d
    x = vals((T, dm), 920, dtype)
    w1 = vals((4 * hd, dm), 921, dtype, 1.0 / np.sqrt(dm))
    b1 = params(4 * hd, 922, 0.1)
    w2 = vals((dm, hd), 923, dtype, 1.0 / np.sqrt(hd))
    gamma, beta, b2 = 1.0 + params(hd, 924, 0.1), params(hd, 925, 0.1), params(dm, 926, 0.1)
    attn = vals((T, H, d), 927, dtype, 0.05)
    xd = to_torch(x, dtype)
    uvqk = hstu.hstu_layer_in_proj(xd, to_torch(w1, dtype), f32dev(b1), H, d)
    y = hstu.hstu_layer_out_proj(to_torch(attn, dtype), uvqk[0], xd, f32dev(gamma), f32dev(beta),
                                 1e-5, to_torch(w2, dtype), f32dev(b2))
    torch.cuda.synchronize()
    ref_in = oracle.layer_in(x, w1, b1.astype(np.float64), H, d, dtype)
    for name, g, r in zip("uvqk", uvqk, ref_in):
        mr, l2 = assert_close(from_torch(g, dtype), r, dtype, f"layer_in {name} whole output")
        log(f"  layer_in {name}: max|err|/max|ref| = {mr:.3e}, rel L2 = {l2:.3e}")
    u_host = from_torch(uvqk[0], dtype)
    u_store = workloads.cast_values(u_host.astype(np.float32), dtype)   # the stored u, exactly
    ref_out = oracle.layer_out(attn, u_store, x, gamma.astype(np.float64),
                               beta.astype(np.float64), float(np.float32(1e-5)), w2,
                               b2.astype(np.float64), H, d, dtype)
    mr, l2 = assert_close(from_torch(y, dtype), ref_out, dtype, "layer_out whole output")
    log(f"  layer_out: max|err|/max|ref| = {mr:.3e}, rel L2 = {l2:.3e}")


def test_layer_end_to_end_small():
    """x -> projections -> attention -> output, against the oracle chain with
    the intermediates rounded to bf16 as the GPU stores them."""
    dtype, dm, H, d = "bf16", 256, 4, 64
    lengths = [100, 0, 257, 33]
    off = workloads.offsets_from_lengths(lengths)
    T = int(off[-1])
    hd = H * d
    x = vals((T, dm), 930, dtype)
    w1 = vals((4 * hd, dm), 931, dtype, 1.0 / np.sqrt(dm))
    b1 = params(4 * hd, 932, 0.1)
    w2 = vals((dm, hd), 933, dtype, 1.0 / np.sqrt(hd))
    gamma, beta, b2 = 1.0 + params(hd, 934, 0.1), params(hd, 935, 0.1), params(dm, 936, 0.1)
    alpha, n, eps = 0.125, 257.0, 1e-5
    xd = to_torch(x, dtype)
    u, v, q, k = hstu.hstu_layer_in_proj(xd, to_torch(w1, dtype), f32dev(b1), H, d)
    offd = torch.from_numpy(off).cuda()
    a = hstu.hstu_attn_fwd(q, k, v, offd, alpha, n)
    y = hstu.hstu_layer_out_proj(a, u, xd, f32dev(gamma), f32dev(beta), eps, to_torch(w2, dtype),
                                 f32dev(b2))
    torch.cuda.synchronize()

    def rnd(z):
        return workloads.cast_values(z.astype(np.float32), dtype)

    ru, rv, rq, rk = (rnd(z) for z in oracle.layer_in(x, w1, b1.astype(np.float64), H, d, dtype))
    ra = rnd(oracle.fwd(rq, rk, rv, off, H, d, alpha, n, dtype))
    ry = oracle.layer_out(ra, ru, x, gamma.astype(np.float64), beta.astype(np.float64),
                          float(np.float32(eps)), w2, b2.astype(np.float64), H, d, dtype)
    mr, l2 = assert_close(from_torch(y, dtype), ry, dtype, "layer end to end")
    log(f"  end to end: max|err|/max|ref| = {mr:.3e}, rel L2 = {l2:.3e}")
