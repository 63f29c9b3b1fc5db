"""Shared helpers for the GPU parity tests and the benchmark's checks."""
from __future__ import annotations

import sys
from typing import Tuple

import numpy as np

import workloads

# Tolerances.  bf16/fp16 inputs: max|err| <= 1e-2 * max|ref| and relative L2 <= 5e-3.
# fp32 inputs: both measures <= 1e-4.
TOL = {"bf16": (1e-2, 5e-3), "fp16": (1e-2, 5e-3), "fp32": (1e-4, 1e-4)}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(dtype: str):
    import torch
    return {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dtype]


def to_torch(x: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device)


def from_torch(t, dtype: str) -> np.ndarray:
    """Stored values of a device tensor, widened exactly to fp64."""
    import torch
    if dtype == "bf16":
        u = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
        return workloads.bf16_bits_to_f32(u).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def device_case(case: workloads.Case, device="cuda"):
    import torch
    q = to_torch(case.q, case.dtype, device)
    k = to_torch(case.k, case.dtype, device)
    v = to_torch(case.v, case.dtype, device)
    off = torch.from_numpy(case.offsets.astype(np.int32)).to(device)
    return q, k, v, off


def errors(got: np.ndarray, ref: np.ndarray) -> Tuple[float, float]:
    """(max|err| / max|ref|, ||err||_2 / ||ref||_2) over all elements."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0, 0.0
    err = got - ref
    mref = float(np.max(np.abs(ref)))
    nref = float(np.linalg.norm(ref))
    max_ratio = float(np.max(np.abs(err))) / mref if mref > 0 else float(np.max(np.abs(err)))
    l2 = float(np.linalg.norm(err)) / nref if nref > 0 else float(np.linalg.norm(err))
    return max_ratio, l2


def assert_close(got, ref, dtype: str, what: str = "") -> Tuple[float, float]:
    max_ratio, l2 = errors(got, ref)
    tmax, tl2 = TOL[dtype]
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert max_ratio <= tmax and l2 <= tl2, (
        f"{what}: max|err|/max|ref| = {max_ratio:.3e} (tol {tmax}), rel L2 = {l2:.3e} (tol {tl2})")
    return max_ratio, l2


def sample_rows(case: workloads.Case, max_seqs: int = 48, per_seq_random: int = 6,
                seed: int = 7):
    """(tokens, heads) to check: tile-boundary rows and random rows of a subset
    of sequences (longest, shortest and random ones), every head."""
    rng = np.random.default_rng(seed)
    L = case.lengths
    nz = np.nonzero(L > 0)[0]
    if len(nz) > max_seqs:
        order = nz[np.argsort(-L[nz], kind="stable")]
        pick = set(order[:max_seqs // 4].tolist()) | set(order[-max_seqs // 4:].tolist())
        rest = [i for i in nz if i not in pick]
        pick |= set(rng.choice(rest, size=max_seqs - len(pick), replace=False).tolist())
        seqs = sorted(pick)
    else:
        seqs = list(nz)
    toks, hds = [], []
    for i in seqs:
        s = int(L[i])
        base = int(case.offsets[i])
        rows = {0, s - 1}
        for b in (32, 64, 128, 256):
            for m in range(1, 4):
                for dlt in (-1, 0, 1):
                    r = b * m + dlt
                    if 0 <= r < s:
                        rows.add(r)
        rows |= set(rng.integers(0, s, size=per_seq_random).tolist())
        for r in sorted(rows):
            for h in range(case.heads):
                toks.append(base + r)
                hds.append(h)
    return np.array(toks, np.int64), np.array(hds, np.int32)
