"""Seeded synthetic inputs for the HSTU jagged attention forward.

This module holds no part of the attention arithmetic.  It only draws
sequence lengths and i.i.d. normal values, rounds them to the element type
the call runs in, and builds int32 prefix-sum offsets.  Both the CPU oracle
(under ``oracle/``) and the HIP library consume what it returns; neither of
them is imported here.

The five named workloads follow the shapes the pages measure:
  * the Ascend HSTU blog ("都是生成式推荐，为什么昇腾这么快？") times
    QKV (b=16, heads=4, s=4096, d=64) in §2.2, §3.2 and §5.2, and bounds real
    lengths by 0 < s <= 20480 in §3.1;
  * the HSTU paper translation ("行动胜于言语…", §3.2) notes that user history
    lengths are skewed, which the skewed-length workload stands in for.
No public dataset is involved; every value is synthetic.

Element types are carried as numpy arrays:
  * "fp32": float32
  * "fp16": float16 (numpy's cast rounds to nearest even)
  * "bf16": uint16 holding bfloat16 bit patterns, rounded to nearest even
    from float32 by the integer rule below.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

DTYPES = ("bf16", "fp16", "fp32")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs here are finite normals, so the NaN/overflow corner of the rounding
    rule does not arise; a NaN input is kept a quiet NaN anyway.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def cast_values(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float32 array to the storage form of `dtype` (see module doc)."""
    if dtype == "fp32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "fp16":
        return np.ascontiguousarray(x32, dtype=np.float32).astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


def widen_to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 image of stored values (for display and sums in tests)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x)
    return np.asarray(x, dtype=np.float32)


def offsets_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    if (lengths < 0).any():
        raise ValueError("negative sequence length")
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    if off[-1] > np.iinfo(np.int32).max:
        raise ValueError("total length does not fit int32 offsets")
    return off.astype(np.int32)


@dataclasses.dataclass
class Case:
    """One synthetic call: jagged q/k/v (T, heads, d) plus offsets and scalars."""

    name: str
    dtype: str
    heads: int
    d: int
    offsets: np.ndarray  # int32 [num_seqs + 1]
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: float  # the float32 value handed to the kernel
    n: float  # the float32 value handed to the kernel
    description: str = ""
    # candidates at the end of each sequence (target-aware mask), or None
    num_targets: Optional[np.ndarray] = None

    @property
    def num_seqs(self) -> int:
        return len(self.offsets) - 1

    @property
    def total(self) -> int:
        return int(self.offsets[-1])

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.offsets.astype(np.int64))

    def useful_flops(self) -> float:
        """4 * heads * d * sum_i s_i (s_i + 1) / 2: both products, causal half
        including the diagonal, nothing for the skipped upper triangle."""
        s = self.lengths.astype(np.float64)
        return float(4.0 * self.heads * self.d * np.sum(s * (s + 1.0) / 2.0))

    def algorithmic_bytes(self) -> float:
        """q, k, v read once and out written once, plus the offsets."""
        elt = {"bf16": 2, "fp16": 2, "fp32": 4}[self.dtype]
        return float(4 * elt * self.total * self.heads * self.d + 4 * (self.num_seqs + 1))


def f32(x: float) -> float:
    """The float32 value nearest to x, as a Python float."""
    return float(np.float32(x))


def make_case(lengths, heads: int, d: int, dtype: str, seed: int, sigma: float = 1.0,
              alpha: Optional[float] = None, n: Optional[float] = None,
              name: str = "custom", description: str = "") -> Case:
    """Jagged case from explicit lengths; values i.i.d. N(0, sigma^2)."""
    if dtype not in DTYPES:
        raise ValueError(dtype)
    offsets = offsets_from_lengths(lengths)
    T = int(offsets[-1])
    rng = np.random.default_rng(seed)
    shape = (T, heads, d)
    vals = []
    for _ in range(3):
        x = rng.standard_normal(shape, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        vals.append(cast_values(x, dtype))
    if alpha is None:
        alpha = 1.0 / math.sqrt(d)
    if n is None:
        n = float(max(1, int(np.max(np.diff(offsets))) if len(offsets) > 1 else 1))
    return Case(name=name, dtype=dtype, heads=heads, d=d, offsets=offsets,
                q=vals[0], k=vals[1], v=vals[2], alpha=f32(alpha), n=f32(n),
                description=description)


# ---------------------------------------------------------------------------
# The five named workloads.  Seed = 1000 + workload number; lengths are drawn
# before values from the same generator.
# ---------------------------------------------------------------------------

WORKLOADS: Dict[int, str] = {
    1: "dense causal, 1 x 256 tokens, heads 2, d 64, fp32",
    2: "dense causal as 16 equal jagged sequences of 4096, heads 4, d 64, bf16",
    3: "jagged causal, 64 skewed lengths max(16, ceil(8192 u^3)), heads 4, d 128, bf16",
    4: "long jagged causal, 8 lengths U[8192, 20480], heads 4, d 64, bf16",
    5: "many short jagged causal, 4096 lengths U[1, 256], heads 2, d 128, fp16",
}


def workload_lengths(num: int, rng: np.random.Generator) -> List[int]:
    if num == 1:
        return [256]
    if num == 2:
        return [4096] * 16
    if num == 3:
        u = rng.random(64)
        return [int(x) for x in np.maximum(16, np.ceil(8192.0 * u ** 3))]
    if num == 4:
        return [int(x) for x in rng.integers(8192, 20480, size=8, endpoint=True)]
    if num == 5:
        return [int(x) for x in rng.integers(1, 256, size=4096, endpoint=True)]
    raise ValueError(f"no workload {num}")


_SPEC = {
    # num: (heads, d, dtype, sigma, alpha, n-rule)
    1: (2, 64, "fp32", 1.0, 1.0 / math.sqrt(64), lambda L: 256.0),
    2: (4, 64, "bf16", 1.0, 1.0 / 8.0, lambda L: 4096.0),
    3: (4, 128, "bf16", 1.0, 1.0 / math.sqrt(128), lambda L: float(max(L))),
    4: (4, 64, "bf16", 1.0, 1.0 / 8.0, lambda L: 20480.0),
    5: (2, 128, "fp16", 0.5, 1.0 / math.sqrt(128), lambda L: 256.0),
}


def workload(num: int, values: bool = True) -> Case:
    """Build named workload `num` (1..5).  With values=False only the lengths,
    offsets and scalars are filled (q/k/v are empty arrays)."""
    heads, d, dtype, sigma, alpha, n_rule = _SPEC[num]
    rng = np.random.default_rng(1000 + num)
    lengths = workload_lengths(num, rng)
    offsets = offsets_from_lengths(lengths)
    T = int(offsets[-1])
    if values:
        vals = []
        for _ in range(3):
            x = rng.standard_normal((T, heads, d), dtype=np.float32)
            if sigma != 1.0:
                x *= np.float32(sigma)
            vals.append(cast_values(x, dtype))
    else:
        empty = cast_values(np.zeros((0, heads, d), np.float32), dtype)
        vals = [empty, empty, empty]
    return Case(name=f"w{num}", dtype=dtype, heads=heads, d=d, offsets=offsets,
                q=vals[0], k=vals[1], v=vals[2], alpha=f32(alpha), n=f32(n_rule(lengths)),
                description=WORKLOADS[num])


# ---------------------------------------------------------------------------
# Ranking with appended candidates (M-FALCON micro-batches, HSTU paper
# translation §3.4 and Appendix H: one micro-batch of b_m candidates follows
# each user's history; Fig. 13 uses b_m = 1024).  Same token count, heads, d
# and scalars as the 16 x 4096 causal workload: 16 users, history 3072,
# 1024 candidates each.  Seed 1100.
# ---------------------------------------------------------------------------

TARGETS_DESCRIPTION = ("target-aware, 16 users x (3072 history + 1024 candidates), "
                       "heads 4, d 64, bf16")


def targets_workload(values: bool = True, history: int = 3072, candidates: int = 1024,
                     users: int = 16) -> Case:
    rng = np.random.default_rng(1100)
    heads, d, dtype = 4, 64, "bf16"
    lengths = [history + candidates] * users
    offsets = offsets_from_lengths(lengths)
    T = int(offsets[-1])
    if values:
        vals = [cast_values(rng.standard_normal((T, heads, d), dtype=np.float32), dtype)
                for _ in range(3)]
    else:
        empty = cast_values(np.zeros((0, heads, d), np.float32), dtype)
        vals = [empty, empty, empty]
    return Case(name="targets", dtype=dtype, heads=heads, d=d, offsets=offsets,
                q=vals[0], k=vals[1], v=vals[2], alpha=f32(1.0 / 8.0),
                n=f32(float(history + candidates)), description=TARGETS_DESCRIPTION,
                num_targets=np.full(users, candidates, dtype=np.int32))


# ---------------------------------------------------------------------------
# Later micro-batches against a cached history (M-FALCON with the
# encoder-level K/V cache, HSTU paper translation Appendix H): 16 users, a
# cached history of 3072 rows each (K and V only), one micro-batch of 1024
# candidates each (q, k, v).  Seed 1200: history K, V, then candidate q, k, v.
# ---------------------------------------------------------------------------

CACHED_DESCRIPTION = ("cached history, 16 users x (3072 cached history rows, "
                      "1024 candidates), heads 4, d 64, bf16")


@dataclasses.dataclass
class CachedCase:
    """Candidates (a Case: q, k, v, offsets) plus the cached history K, V and
    their offsets."""

    cand: Case
    k_cache: np.ndarray
    v_cache: np.ndarray
    hist_offsets: np.ndarray  # int32 [num_seqs + 1]

    @property
    def hist_lengths(self) -> np.ndarray:
        return np.diff(self.hist_offsets.astype(np.int64))


def make_cached_case(hist_lengths, cand_lengths, heads: int, d: int, dtype: str, seed: int,
                     sigma: float = 1.0, alpha: Optional[float] = None,
                     n: Optional[float] = None) -> CachedCase:
    """History K, V then candidate q, k, v, i.i.d. N(0, sigma^2), one generator."""
    if len(hist_lengths) != len(cand_lengths):
        raise ValueError("one history length per request")
    rng = np.random.default_rng(seed)
    hoff = offsets_from_lengths(hist_lengths)
    coff = offsets_from_lengths(cand_lengths)

    def draw(rows):
        x = rng.standard_normal((rows, heads, d), dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        return cast_values(x, dtype)

    kc, vc = draw(int(hoff[-1])), draw(int(hoff[-1]))
    q, k, v = draw(int(coff[-1])), draw(int(coff[-1])), draw(int(coff[-1]))
    if alpha is None:
        alpha = 1.0 / math.sqrt(d)
    if n is None:
        n = float(max([1] + [int(a) + int(b) for a, b in zip(hist_lengths, cand_lengths)]))
    cand = Case(name="cached", dtype=dtype, heads=heads, d=d, offsets=coff, q=q, k=k, v=v,
                alpha=f32(alpha), n=f32(n))
    return CachedCase(cand=cand, k_cache=kc, v_cache=vc, hist_offsets=hoff)


def cached_workload(history: int = 3072, candidates: int = 1024, users: int = 16) -> CachedCase:
    c = make_cached_case([history] * users, [candidates] * users, 4, 64, "bf16", seed=1200,
                         alpha=1.0 / 8.0, n=float(history + candidates))
    c.cand.description = CACHED_DESCRIPTION
    return c


# ---------------------------------------------------------------------------
# Relative attention bias inputs: token timestamps and the two bias tables.
# ---------------------------------------------------------------------------

RAB_DESCRIPTION = ("causal with relative attention bias, 16 x 4096, heads 4, d 64, bf16, "
                   "4096 position entries, 16 time buckets")


@dataclasses.dataclass
class RabInputs:
    """int32 timestamps, one per token, and float32 position / time tables."""

    timestamps: np.ndarray  # int32 [T]
    pos_bias: np.ndarray    # float32 [npos]
    time_bias: np.ndarray   # float32 [ntime]


def make_rab_inputs(offsets, npos: int, ntime: int, seed: int, sigma: float = 0.5,
                    max_log_gap: int = 16) -> RabInputs:
    """Per sequence, a start time drawn uniformly in [0, 2^30) and then gaps
    floor(2^(u * max_log_gap)) - 1, u ~ U(0, 1), between consecutive tokens
    (non-decreasing timestamps whose gaps spread over every log2 bucket up to
    max_log_gap); tables i.i.d. N(0, sigma^2)."""
    rng = np.random.default_rng(seed)
    off = np.asarray(offsets, dtype=np.int64)
    T = int(off[-1]) if len(off) else 0
    ts = np.zeros(T, dtype=np.int64)
    for i in range(len(off) - 1):
        a, b = int(off[i]), int(off[i + 1])
        if b == a:
            continue
        gaps = np.floor(np.exp2(rng.random(b - a - 1) * max_log_gap)).astype(np.int64) - 1
        ts[a] = rng.integers(0, 1 << 30)
        ts[a + 1:b] = ts[a] + np.cumsum(gaps)
    if T and ts.max() >= (1 << 31) - 1:
        raise ValueError("timestamps overflow int32; use shorter sequences or smaller gaps")
    wpos = (rng.standard_normal(npos, dtype=np.float32) * np.float32(sigma)).astype(np.float32)
    wtime = (rng.standard_normal(ntime, dtype=np.float32) * np.float32(sigma)).astype(np.float32)
    return RabInputs(timestamps=ts.astype(np.int32), pos_bias=wpos, time_bias=wtime)


def make_cached_rab_inputs(hist_offsets, cand_offsets, npos: int, ntime: int, seed: int,
                           sigma: float = 0.5, max_log_gap: int = 16):
    """Timestamps for the cached-history form: per request, one timeline as in
    make_rab_inputs over its history followed by its candidates, split into the
    history's (hist_ts, the layout of the cache) and the candidates'
    (cand_ts, the layout of q).  Returns (RabInputs with the candidates'
    timestamps, hist_ts)."""
    hoff = np.asarray(hist_offsets, dtype=np.int64)
    coff = np.asarray(cand_offsets, dtype=np.int64)
    hl, cl = np.diff(hoff), np.diff(coff)
    joint = offsets_from_lengths((hl + cl).tolist())
    r = make_rab_inputs(joint, npos, ntime, seed, sigma=sigma, max_log_gap=max_log_gap)
    hts = np.zeros(int(hoff[-1]) if len(hoff) else 0, dtype=np.int32)
    cts = np.zeros(int(coff[-1]) if len(coff) else 0, dtype=np.int32)
    for i in range(len(hl)):
        j0 = int(joint[i])
        hts[hoff[i]:hoff[i + 1]] = r.timestamps[j0:j0 + hl[i]]
        cts[coff[i]:coff[i + 1]] = r.timestamps[j0 + hl[i]:j0 + hl[i] + cl[i]]
    return RabInputs(timestamps=cts, pos_bias=r.pos_bias, time_bias=r.time_bias), hts


def rab_workload(values: bool = True):
    """The causal workload of 16 sequences of 4096 tokens (heads 4, d 64,
    bf16) with a relative attention bias: a position entry per distance and
    16 time buckets.  Seed 1300."""
    case = make_case([4096] * 16, 4, 64, "bf16", seed=1300, alpha=1.0 / 8.0, n=4096.0,
                     name="rab", description=RAB_DESCRIPTION) if values else None
    offsets = case.offsets if case is not None else offsets_from_lengths([4096] * 16)
    return case, make_rab_inputs(offsets, 4096, 16, seed=1301)


def rab_cached_workload():
    """The cached-history workload (16 x (3072 cached + 1024 candidates),
    heads 4, d 64, bf16) with a relative attention bias: a position entry per
    distance and 16 time buckets.  Seeds 1200 (K, V, q, k, v) and 1321 (bias).
    Returns (CachedCase, RabInputs with the candidates' timestamps, the
    history's timestamps)."""
    cc = cached_workload()
    r, hts = make_cached_rab_inputs(cc.hist_offsets, cc.cand.offsets, 4096, 16, seed=1321)
    return cc, r, hts


def rab_targets_workload(values: bool = True):
    """The target-aware workload (16 x (3072 history + 1024 candidates),
    heads 4, d 64, bf16) with a relative attention bias: a position entry per
    distance and 16 time buckets.  Seeds 1100 (q, k, v) and 1311 (bias)."""
    case = targets_workload(values)
    return case, make_rab_inputs(case.offsets, 4096, 16, seed=1311)
