"""Pins for the oracle's backward (gradients of the forward with respect to q,
k and v).

The pages only say that the backward recomputes the attention instead of
storing it (HSTU paper translation, Appendix G); the gradients are the
derivative of the forward definition (Ascend HSTU blog, §1).  Each pin raises
AssertionError when the oracle disagrees with something fixed independently of
its code: central finite differences of the forward, torch's automatic
differentiation of a dense float64 forward, the closed form of a one-token
sequence, or the identity <dv, v> = <dout, out> (out is linear in v).
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads


def _case(lengths, heads, d, seed, targets=None, alpha=0.7, n=3.0):
    c = workloads.make_case(lengths, heads, d, "fp32", seed=seed, alpha=alpha, n=n)
    dout = workloads.make_case(lengths, heads, d, "fp32", seed=seed + 1).q
    return c, dout, targets


def _dense_loss(q, k, v, dout, offsets, heads, d, alpha, n, targets):
    """sum(dout * out) with out from the numpy dense evaluation (float64 in)."""
    out = oracle.dense_pairs(q, k, v, offsets, heads, d, alpha, n, "fp32",
                               num_targets=targets)
    return float(np.sum(dout * out))


def pin_bwd_finite_differences(lib) -> None:
    """Central differences of sum(dout * out) over every input element."""
    for lengths, targets in (([3, 4], None), ([5, 2], [2, 1])):
        c, dout, tg = _case(lengths, 2, 3, seed=101, targets=targets)
        dq, dk, dv = oracle.bwd(c.q, c.k, c.v, dout, c.offsets, 2, 3, c.alpha, c.n, "fp32",
                                lib=lib, num_targets=tg)
        base = [c.q.astype(np.float64), c.k.astype(np.float64), c.v.astype(np.float64)]
        do = dout.astype(np.float64)
        h = 1e-5
        for which, grad in enumerate((dq, dk, dv)):
            fd = np.zeros_like(grad)
            for idx in np.ndindex(*grad.shape):
                vals = []
                for sgn in (1.0, -1.0):
                    args = [b.copy() for b in base]
                    args[which][idx] += sgn * h
                    vals.append(_dense_loss(*args, do, c.offsets, 2, 3, c.alpha, c.n, tg))
                fd[idx] = (vals[0] - vals[1]) / (2 * h)
            err = np.max(np.abs(fd - grad))
            assert err <= 1e-7 * max(1.0, float(np.max(np.abs(grad)))), ("qkv"[which], err)


def pin_bwd_autograd(lib) -> None:
    """torch autograd (CPU, float64) of the dense forward, per sequence."""
    import torch
    c, dout, _ = _case([6, 1, 9], 2, 5, seed=111)
    dq, dk, dv = oracle.bwd(c.q, c.k, c.v, dout, c.offsets, 2, 5, c.alpha, c.n, "fp32",
                            lib=lib)
    for i in range(c.num_seqs):
        a, b = int(c.offsets[i]), int(c.offsets[i + 1])
        Q, K, V = (torch.tensor(x[a:b].astype(np.float64).transpose(1, 0, 2), requires_grad=True)
                   for x in (c.q, c.k, c.v))
        S = c.alpha * torch.matmul(Q, K.transpose(1, 2))
        mask = torch.tril(torch.ones(b - a, b - a, dtype=torch.float64))
        out = torch.matmul(torch.nn.functional.silu(S) * mask / c.n, V)
        out.backward(torch.tensor(dout[a:b].astype(np.float64).transpose(1, 0, 2)))
        for got, ref in ((dq, Q.grad), (dk, K.grad), (dv, V.grad)):
            r = ref.numpy().transpose(1, 0, 2)
            assert np.max(np.abs(got[a:b] - r)) <= 1e-12 * max(1.0, float(np.max(np.abs(r))))


def pin_bwd_one_token(lib) -> None:
    """One-token sequences: out = silu(x) v / n with x = alpha <q, k>, so
    dv = silu(x) dout / n and dq = (alpha/n) silu'(x) <dout, v> k (dk with q),
    silu'(x) = (1 + e^-x + x e^-x) / (1 + e^-x)^2."""
    c, dout, _ = _case([1, 1, 1], 3, 4, seed=121, alpha=0.9, n=2.0)
    dq, dk, dv = oracle.bwd(c.q, c.k, c.v, dout, c.offsets, 3, 4, c.alpha, c.n, "fp32",
                            lib=lib)
    q, k, v, do = (x.astype(np.float64) for x in (c.q, c.k, c.v, dout))
    x = c.alpha * np.sum(q * k, axis=-1, keepdims=True)
    em = np.exp(-x)
    silu = x / (1.0 + em)
    dsilu = (1.0 + em + x * em) / (1.0 + em) ** 2
    dov = np.sum(do * v, axis=-1, keepdims=True)
    for got, ref in ((dv, silu * do / c.n), (dq, c.alpha / c.n * dsilu * dov * k),
                     (dk, c.alpha / c.n * dsilu * dov * q)):
        assert np.max(np.abs(got - ref)) <= 1e-13 * max(1.0, float(np.max(np.abs(ref))))


def pin_bwd_value_identity(lib) -> None:
    """out is linear in v, so <dv, v> = sum(dout * out) (the forward oracle),
    with either mask."""
    for tg in (None, [3, 0, 5]):
        c, dout, _ = _case([7, 4, 6], 2, 8, seed=131)
        _, _, dv = oracle.bwd(c.q, c.k, c.v, dout, c.offsets, 2, 8, c.alpha, c.n, "fp32",
                              lib=lib, num_targets=tg)
        out = oracle.fwd(c.q, c.k, c.v, c.offsets, 2, 8, c.alpha, c.n, "fp32", lib=lib,
                         num_targets=tg)
        lhs = float(np.sum(dv * c.v.astype(np.float64)))
        rhs = float(np.sum(dout.astype(np.float64) * out))
        assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(rhs)), (lhs, rhs)


def pin_bwd_rows_match(lib) -> None:
    """Sampled gradient rows equal the full gradients' rows (bf16 storage)."""
    c = workloads.make_case([9, 0, 13], 2, 64, "bf16", seed=141)
    dout = workloads.make_case([9, 0, 13], 2, 64, "bf16", seed=142).q
    tg = [4, 0, 6]
    full = oracle.bwd(c.q, c.k, c.v, dout, c.offsets, 2, 64, c.alpha, c.n, "bf16", lib=lib,
                      num_targets=tg)
    toks = np.array([0, 5, 8, 9, 15, 21], dtype=np.int64)
    hds = np.array([1, 0, 1, 0, 1, 0], dtype=np.int32)
    for kind, g in zip(("dq", "dk", "dv"), full):
        r = oracle.bwd_rows(c.q, c.k, c.v, dout, c.offsets, 2, 64, c.alpha, c.n, "bf16", kind,
                            toks, hds, lib=lib, num_targets=tg)
        assert np.array_equal(r, g[toks, hds]), kind


BWD_PINS = [pin_bwd_finite_differences, pin_bwd_autograd, pin_bwd_one_token,
            pin_bwd_value_identity, pin_bwd_rows_match]
