"""Pins for the oracle's layer surroundings (HSTU paper translation §3, §3.3):
[u | v | q | k] = silu(W1 x + b1) per token, and y = x + W2 (LN(a) * u) + b2
with LN the layer normalisation over heads * d.

Each pin raises AssertionError when the oracle disagrees with something fixed
independently of its loops: one-hot weights that read single input columns
(closed forms that fix the split order and the layout), torch's float64
matmul / silu / layer_norm, and the normalisation's own invariants.
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads


def _vals(shape, seed, dtype="fp32", scale=1.0):
    rng = np.random.default_rng(seed)
    return workloads.cast_values((rng.standard_normal(shape) * scale).astype(np.float32), dtype)


def _silu(z):
    return z / (1.0 + np.exp(-z))


def pin_layer_in_one_hot(lib) -> None:
    """W1 row c reads input column c % d_model: every output is silu of one
    input plus its bias, which fixes the split order (u, v, q, k) and the
    (heads, d) layout of each part."""
    T, dm, H, d = 3, 32, 2, 4
    hd = H * d
    x = _vals((T, dm), 1)
    w1 = np.zeros((4 * hd, dm), np.float32)
    for c in range(4 * hd):
        w1[c, c % dm] = 1.0
    b1 = np.arange(4 * hd) * 0.01
    got = oracle.layer_in(x, w1, b1, H, d, "fp32", lib=lib)
    xf = x.astype(np.float64)
    for part in range(4):
        for h in range(H):
            for e in range(d):
                c = part * hd + h * d + e
                ref = _silu(xf[:, c % dm] + b1[c])
                assert np.allclose(got[part][:, h, e], ref, rtol=0, atol=1e-15), (part, h, e)


def pin_layer_in_torch(lib) -> None:
    """Against torch float64: silu(x @ w1.T + b1), split in four."""
    import torch
    T, dm, H, d = 7, 64, 2, 16
    x, w1 = _vals((T, dm), 2, "bf16"), _vals((4 * H * d, dm), 3, "bf16", 0.2)
    b1 = np.random.default_rng(4).standard_normal(4 * H * d)
    got = oracle.layer_in(x, w1, b1, H, d, "bf16", lib=lib)
    xt = torch.tensor(oracle.widen(x, "bf16"))
    wt = torch.tensor(oracle.widen(w1, "bf16"))
    ref = torch.nn.functional.silu(xt @ wt.T + torch.tensor(b1)).numpy()
    for part in range(4):
        r = ref[:, part * H * d:(part + 1) * H * d].reshape(T, H, d)
        assert np.max(np.abs(got[part] - r)) <= 1e-13


def pin_layer_out_torch(lib) -> None:
    """Against torch float64: x + (layer_norm(a) * u) @ w2.T + b2."""
    import torch
    T, dm, H, d = 6, 48, 4, 8
    hd = H * d
    attn, u = _vals((T, H, d), 5, "fp16", 0.3), _vals((T, H, d), 6, "fp16")
    x, w2 = _vals((T, dm), 7, "fp16"), _vals((dm, hd), 8, "fp16", 0.2)
    rng = np.random.default_rng(9)
    gamma, beta, b2 = rng.standard_normal(hd), rng.standard_normal(hd), rng.standard_normal(dm)
    eps = 1e-5
    got = oracle.layer_out(attn, u, x, gamma, beta, eps, w2, b2, H, d, "fp16", lib=lib)
    a = torch.tensor(oracle.widen(attn, "fp16").reshape(T, hd))
    ln = torch.nn.functional.layer_norm(a, (hd,), torch.tensor(gamma), torch.tensor(beta), eps)
    z = ln * torch.tensor(oracle.widen(u, "fp16").reshape(T, hd))
    ref = (torch.tensor(oracle.widen(x, "fp16")) + z @ torch.tensor(oracle.widen(w2, "fp16")).T
           + torch.tensor(b2)).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, float(np.max(np.abs(ref))))


def pin_layer_out_closed_forms(lib) -> None:
    """u = 0 gives y = x + b2 exactly; with u = 1, gamma = 1, beta = 0 and
    W2 = I (d_model = heads d), y - x - b2 is the normalised row: mean 0 and
    mean square var / (var + eps)."""
    T, H, d = 5, 2, 8
    hd = H * d
    attn = _vals((T, H, d), 11, scale=2.0)
    x = _vals((T, hd), 12)
    b2 = np.linspace(-1, 1, hd)
    w2 = np.eye(hd, dtype=np.float32)
    zero = np.zeros((T, H, d), np.float32)
    one = np.ones((T, H, d), np.float32)
    eps = 1e-3
    y0 = oracle.layer_out(attn, zero, x, np.ones(hd), np.zeros(hd), eps, w2, b2, H, d, "fp32",
                          lib=lib)
    assert np.array_equal(y0, x.astype(np.float64) + b2)
    y1 = oracle.layer_out(attn, one, x, np.ones(hd), np.zeros(hd), eps, w2, b2, H, d, "fp32",
                          lib=lib)
    ln = y1 - x.astype(np.float64) - b2
    a = attn.astype(np.float64).reshape(T, hd)
    var = a.var(axis=1)
    assert np.allclose(ln.mean(axis=1), 0.0, atol=1e-12)
    assert np.allclose((ln ** 2).mean(axis=1), var / (var + eps), rtol=1e-12, atol=0)


LAYER_PINS = [pin_layer_in_one_hot, pin_layer_in_torch, pin_layer_out_torch,
              pin_layer_out_closed_forms]
