"""CPU oracle for the HSTU jagged causal attention forward.

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP library and
its Python binding never import it, and it imports nothing from them: the two
share no code.  The only module both sides read is ``workloads`` (seeded input
generation, no attention arithmetic).

Two independent evaluations of the same definition live here:

* ``fwd`` / ``rows``: the plain row-by-row fp64 loop in ``hstu_oracle.c``
  (OpenMP over (sequence, head) pairs), built with gcc;
* ``dense_pairs``: numpy fp64, one sequence at a time, written from the
  definition as a sum over kept (row, key) pairs: a boolean matrix says which
  keys each row sees (key <= row for the causal mask, the Ascend HSTU blog
  "都是生成式推荐，为什么昇腾这么快？" §3.1-§3.2), every score of a kept pair
  is formed with einsum, weighted by silu(alpha * score), and the weighted
  values of a row's kept keys are summed and divided by n.  Jagged packing
  follows §4.2 of that page.

The ``num_targets`` arguments give the target-aware (M-FALCON) mask of the
HSTU paper translation (§3.4, Appendix H, Algorithm 1 and Fig. 11): the last
t tokens of a sequence are candidates that see the history and themselves
only.  ``num_targets=None`` is the plain causal mask.

``fwd_cached`` / ``rows_cached`` are the later micro-batches of the same
algorithm (Appendix H, the encoder-level K/V cache): candidates with their own
q, k, v attend to a cached history's K and V plus themselves, each request's
history and candidates given by their own offsets; ``fwd_rab_cached`` /
``rows_rab_cached`` add the relative attention bias to that form (a candidate
right after its history, real timestamps).

``bwd`` / ``bwd_rows`` are the gradients with respect to q, k and v: the
derivative of the forward definition, per kept (row, key) pair, for an
upstream gradient dout (the pages only say that the backward recomputes the
attention instead of storing it, HSTU paper translation Appendix G).

``fwd_rab`` / ``rows_rab`` add the relative attention bias rab_{p,t} (HSTU
paper translation §3 and Appendix G) to the scaled score before SiLU, under
the causal mask: rab(r, c) = wpos[r - c] (0 from npos on) +
wtime[min(floor(log2(ts_r - ts_c + 1)), ntime - 1)] (a negative gap in the
last bucket), the tables shared by all heads; ``bwd_rab`` / ``bwd_rab_rows``
are its gradients, the tables' included, under either mask.

``layer_in`` / ``layer_out`` are the layer's surroundings (HSTU paper
translation §3, §3.3): [u | v | q | k] = silu(W1 x + b1) per token, and
y = x + W2 (LN(a) * u) + b2 with LN over heads * d.

Parity status: pinned.  The test suite ties these functions to closed forms
(hand-worked 2- and 3-token cases), to identities that reduce to textbook
operations (sign-flip -> masked GEMM, constant rows -> prefix sum, row 0),
and to invariants (linearity, causality, segment independence); the bias
form also to a plain forward with extra head dimensions and to buckets found
by floating-point log2.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "hstu_oracle.c")
LIBRARY = os.path.join(HERE, "libhstu_oracle.so")

_DTYPE_CODE = {"bf16": 0, "fp16": 1, "fp32": 2}


def build(output: str = LIBRARY, plant: int = 0) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP).  `plant` != 0 builds a
    copy with one deliberate mistake (see the C source) for pin tests."""
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
           f"-DORACLE_PLANT={int(plant)}", SOURCE, "-o", output + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


_libs = {}


def load(path: Optional[str] = None) -> ctypes.CDLL:
    path = path or LIBRARY
    if path in _libs:
        return _libs[path]
    if path == LIBRARY and (not os.path.exists(path)
                            or os.path.getmtime(path) < os.path.getmtime(SOURCE)):
        build(path)
    lib = ctypes.CDLL(path)
    vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.hstu_oracle_fwd.argtypes = [vp, vp, vp, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, f64, f64, vp]
    lib.hstu_oracle_fwd.restype = ctypes.c_int
    lib.hstu_oracle_rows.argtypes = [vp, vp, vp, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, f64, f64, vp, vp, i64, vp]
    lib.hstu_oracle_rows.restype = ctypes.c_int
    lib.hstu_oracle_fwd_targets.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, f64, f64, vp]
    lib.hstu_oracle_fwd_targets.restype = ctypes.c_int
    lib.hstu_oracle_rows_targets.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, f64, f64, vp, vp, i64,
                                             vp]
    lib.hstu_oracle_rows_targets.restype = ctypes.c_int
    lib.hstu_oracle_fwd_cached.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, vp, vp,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int, f64, f64, vp]
    lib.hstu_oracle_fwd_cached.restype = ctypes.c_int
    lib.hstu_oracle_rows_cached.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, vp, vp,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_int, f64, f64,
                                            vp, vp, i64, vp]
    lib.hstu_oracle_rows_cached.restype = ctypes.c_int
    lib.hstu_oracle_bwd.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, f64, f64, vp, vp, vp]
    lib.hstu_oracle_bwd.restype = ctypes.c_int
    lib.hstu_oracle_bwd_rows.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, f64, f64, ctypes.c_int, vp,
                                         vp, i64, vp]
    lib.hstu_oracle_bwd_rows.restype = ctypes.c_int
    lib.hstu_oracle_layer_in.argtypes = [vp, vp, vp, ctypes.c_int, i64, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, vp, vp, vp, vp]
    lib.hstu_oracle_layer_in.restype = ctypes.c_int
    lib.hstu_oracle_layer_out.argtypes = [vp, vp, vp, vp, vp, f64, vp, vp, ctypes.c_int, i64,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    lib.hstu_oracle_layer_out.restype = ctypes.c_int
    lib.hstu_oracle_fwd_rab.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, vp, ctypes.c_int, vp,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        f64, f64, vp]
    lib.hstu_oracle_fwd_rab.restype = ctypes.c_int
    lib.hstu_oracle_rows_rab.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, vp, ctypes.c_int, vp,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         f64, f64, vp, vp, i64, vp]
    lib.hstu_oracle_rows_rab.restype = ctypes.c_int
    lib.hstu_oracle_fwd_rab_targets.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, vp, vp,
                                                ctypes.c_int, vp, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int, ctypes.c_int, f64, f64, vp]
    lib.hstu_oracle_fwd_rab_targets.restype = ctypes.c_int
    lib.hstu_oracle_rows_rab_targets.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, vp, vp,
                                                 ctypes.c_int, vp, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int, ctypes.c_int, f64, f64, vp, vp,
                                                 i64, vp]
    lib.hstu_oracle_rows_rab_targets.restype = ctypes.c_int
    lib.hstu_oracle_bwd_rab.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, ctypes.c_int, vp,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        f64, f64, vp, vp, vp, vp, vp]
    lib.hstu_oracle_bwd_rab.restype = ctypes.c_int
    lib.hstu_oracle_bwd_rab_rows.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, vp, vp,
                                             ctypes.c_int, vp, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, f64, f64, ctypes.c_int,
                                             vp, vp, i64, vp]
    lib.hstu_oracle_bwd_rab_rows.restype = ctypes.c_int
    lib.hstu_oracle_fwd_rab_cached.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, vp,
                                               vp, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, f64, f64, vp]
    lib.hstu_oracle_fwd_rab_cached.restype = ctypes.c_int
    lib.hstu_oracle_rows_rab_cached.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, vp,
                                                vp, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int, ctypes.c_int, f64, f64, vp, vp, i64,
                                                vp]
    lib.hstu_oracle_rows_rab_cached.restype = ctypes.c_int
    lib.hstu_oracle_bwd_rab_targets.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, vp,
                                                ctypes.c_int, vp, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int, ctypes.c_int, f64, f64, vp, vp, vp,
                                                vp, vp]
    lib.hstu_oracle_bwd_rab_targets.restype = ctypes.c_int
    lib.hstu_oracle_bwd_rab_rows_targets.argtypes = [vp, vp, vp, vp, ctypes.c_int, vp, vp, vp,
                                                     vp, ctypes.c_int, vp, ctypes.c_int,
                                                     ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                     f64, f64, ctypes.c_int, vp, vp, i64, vp]
    lib.hstu_oracle_bwd_rab_rows_targets.restype = ctypes.c_int
    lib.hstu_oracle_threads.argtypes = []
    lib.hstu_oracle_threads.restype = ctypes.c_int
    _libs[path] = lib
    return lib


def _storage(x: np.ndarray, dtype: str) -> np.ndarray:
    want = {"bf16": np.uint16, "fp16": np.float16, "fp32": np.float32}[dtype]
    x = np.ascontiguousarray(x)
    if x.dtype != want:
        raise TypeError(f"{dtype} values must be stored as {np.dtype(want).name}, got {x.dtype}")
    return x


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _targets(num_targets, num_seqs: int):
    if num_targets is None:
        return None
    t = np.ascontiguousarray(num_targets, dtype=np.int32)
    if t.shape != (num_seqs,):
        raise ValueError("num_targets needs one count per sequence")
    return t


def fwd(q, k, v, offsets, heads: int, d: int, alpha: float, n: float, dtype: str,
        lib: Optional[ctypes.CDLL] = None, num_targets=None) -> np.ndarray:
    """Full fp64 output (T, heads, d)."""
    lib = lib or load()
    q, k, v = (_storage(a, dtype) for a in (q, k, v))
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    tg = _targets(num_targets, len(off) - 1)
    T = int(off[-1]) if len(off) else 0
    out = np.zeros((T, heads, d), dtype=np.float64)
    for a in (q, k, v):
        if a.size < T * heads * d:
            raise ValueError("q/k/v smaller than offsets imply")
    rc = lib.hstu_oracle_fwd_targets(_ptr(q), _ptr(k), _ptr(v), _DTYPE_CODE[dtype], _ptr(off),
                                     None if tg is None else _ptr(tg), len(off) - 1, heads, d,
                                     float(alpha), float(n), _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (malformed offsets or sizes)")
    return out


def rows(q, k, v, offsets, heads: int, d: int, alpha: float, n: float, dtype: str,
         tokens, head_ids, lib: Optional[ctypes.CDLL] = None, num_targets=None) -> np.ndarray:
    """fp64 outputs (m, d) at global tokens[m], heads head_ids[m]."""
    lib = lib or load()
    q, k, v = (_storage(a, dtype) for a in (q, k, v))
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    tg = _targets(num_targets, len(off) - 1)
    tok = np.ascontiguousarray(tokens, dtype=np.int64)
    hd = np.ascontiguousarray(head_ids, dtype=np.int32)
    if tok.shape != hd.shape:
        raise ValueError("tokens and head_ids differ in length")
    out = np.zeros((len(tok), d), dtype=np.float64)
    rc = lib.hstu_oracle_rows_targets(_ptr(q), _ptr(k), _ptr(v), _DTYPE_CODE[dtype], _ptr(off),
                                      None if tg is None else _ptr(tg), len(off) - 1, heads, d,
                                      float(alpha), float(n), _ptr(tok), _ptr(hd), len(tok),
                                      _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the sampled rows")
    return out


def _cached_args(q, k, v, k_cache, v_cache, cand_offsets, hist_offsets, heads, d, dtype):
    q, k, v, kc, vc = (_storage(a, dtype) for a in (q, k, v, k_cache, v_cache))
    coff = np.ascontiguousarray(cand_offsets, dtype=np.int32)
    hoff = np.ascontiguousarray(hist_offsets, dtype=np.int32)
    if coff.shape != hoff.shape or len(coff) < 1:
        raise ValueError("candidate and history offsets need num_seqs + 1 entries each")
    Tc, Th = int(coff[-1]), int(hoff[-1])
    for a in (q, k, v):
        if a.size < Tc * heads * d:
            raise ValueError("q/k/v smaller than the candidate offsets imply")
    for a in (kc, vc):
        if a.size < Th * heads * d:
            raise ValueError("cached k/v smaller than the history offsets imply")
    return q, k, v, kc, vc, coff, hoff


def fwd_cached(q, k, v, cand_offsets, k_cache, v_cache, hist_offsets, heads: int, d: int,
               alpha: float, n: float, dtype: str,
               lib: Optional[ctypes.CDLL] = None) -> np.ndarray:
    """Full fp64 output (Tc, heads, d) of the candidates against a cached history."""
    lib = lib or load()
    q, k, v, kc, vc, coff, hoff = _cached_args(q, k, v, k_cache, v_cache, cand_offsets,
                                               hist_offsets, heads, d, dtype)
    out = np.zeros((int(coff[-1]), heads, d), dtype=np.float64)
    rc = lib.hstu_oracle_fwd_cached(_ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc),
                                    _DTYPE_CODE[dtype], _ptr(coff), _ptr(hoff), len(coff) - 1,
                                    heads, d, float(alpha), float(n), _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (malformed offsets or sizes)")
    return out


def rows_cached(q, k, v, cand_offsets, k_cache, v_cache, hist_offsets, heads: int, d: int,
                alpha: float, n: float, dtype: str, tokens, head_ids,
                lib: Optional[ctypes.CDLL] = None) -> np.ndarray:
    """fp64 outputs (m, d) of candidate rows tokens[m] (global), heads head_ids[m]."""
    lib = lib or load()
    q, k, v, kc, vc, coff, hoff = _cached_args(q, k, v, k_cache, v_cache, cand_offsets,
                                               hist_offsets, heads, d, dtype)
    tok = np.ascontiguousarray(tokens, dtype=np.int64)
    hd = np.ascontiguousarray(head_ids, dtype=np.int32)
    if tok.shape != hd.shape:
        raise ValueError("tokens and head_ids differ in length")
    out = np.zeros((len(tok), d), dtype=np.float64)
    rc = lib.hstu_oracle_rows_cached(_ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc),
                                     _DTYPE_CODE[dtype], _ptr(coff), _ptr(hoff), len(coff) - 1,
                                     heads, d, float(alpha), float(n), _ptr(tok), _ptr(hd),
                                     len(tok), _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the sampled rows")
    return out


def bwd(q, k, v, dout, offsets, heads: int, d: int, alpha: float, n: float, dtype: str,
        lib: Optional[ctypes.CDLL] = None, num_targets=None):
    """(dq, dk, dv), each fp64 (T, heads, d), for upstream gradient dout."""
    lib = lib or load()
    q, k, v, dout = (_storage(a, dtype) for a in (q, k, v, dout))
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    tg = _targets(num_targets, len(off) - 1)
    T = int(off[-1]) if len(off) else 0
    for a in (q, k, v, dout):
        if a.size < T * heads * d:
            raise ValueError("q/k/v/dout smaller than offsets imply")
    dq, dk, dv = (np.zeros((T, heads, d), dtype=np.float64) for _ in range(3))
    rc = lib.hstu_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _DTYPE_CODE[dtype],
                             _ptr(off), None if tg is None else _ptr(tg), len(off) - 1, heads, d,
                             float(alpha), float(n), _ptr(dq), _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (malformed offsets or sizes)")
    return dq, dk, dv


def _rab_args(q, k, v, offsets, timestamps, pos_bias, time_bias, heads, d, dtype):
    q, k, v = (_storage(a, dtype) for a in (q, k, v))
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    T = int(off[-1]) if len(off) else 0
    ts = np.ascontiguousarray(timestamps, dtype=np.int32)
    wp = np.ascontiguousarray(pos_bias, dtype=np.float64)
    wt = np.ascontiguousarray(time_bias, dtype=np.float64)
    for a in (q, k, v):
        if a.size < T * heads * d:
            raise ValueError("q/k/v smaller than offsets imply")
    if ts.shape != (T,):
        raise ValueError("one timestamp per token")
    if wp.ndim != 1 or wt.ndim != 1:
        raise ValueError("bias tables are 1-D")
    return q, k, v, off, ts, wp, wt


def _rab_cached_args(q, k, v, k_cache, v_cache, cand_offsets, hist_offsets, timestamps,
                     hist_timestamps, pos_bias, time_bias, heads, d, dtype):
    q, k, v, kc, vc, coff, hoff = _cached_args(q, k, v, k_cache, v_cache, cand_offsets,
                                               hist_offsets, heads, d, dtype)
    ts = np.ascontiguousarray(timestamps, dtype=np.int32)
    hts = np.ascontiguousarray(hist_timestamps, dtype=np.int32)
    if ts.size < int(coff[-1]) or hts.size < int(hoff[-1]):
        raise ValueError("timestamps shorter than the offsets imply")
    wp = np.ascontiguousarray(pos_bias, dtype=np.float64)
    wt = np.ascontiguousarray(time_bias, dtype=np.float64)
    return q, k, v, kc, vc, coff, hoff, ts, hts, wp, wt


def fwd_rab_cached(q, k, v, cand_offsets, k_cache, v_cache, hist_offsets, timestamps,
                   hist_timestamps, pos_bias, time_bias, heads: int, d: int, alpha: float,
                   n: float, dtype: str, lib: Optional[ctypes.CDLL] = None) -> np.ndarray:
    """fp64 (T, heads, d): the cached-history form with the relative attention
    bias; timestamps per candidate token, hist_timestamps per cached token."""
    lib = lib or load()
    q, k, v, kc, vc, coff, hoff, ts, hts, wp, wt = _rab_cached_args(
            q, k, v, k_cache, v_cache, cand_offsets, hist_offsets, timestamps, hist_timestamps,
            pos_bias, time_bias, heads, d, dtype)
    out = np.zeros((int(coff[-1]), heads, d), dtype=np.float64)
    rc = lib.hstu_oracle_fwd_rab_cached(_ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc),
                                        _DTYPE_CODE[dtype], _ptr(coff), _ptr(hoff), _ptr(ts),
                                        _ptr(hts), _ptr(wp), len(wp), _ptr(wt), len(wt),
                                        len(coff) - 1, heads, d, float(alpha), float(n),
                                        _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (malformed offsets or sizes)")
    return out


def rows_rab_cached(q, k, v, cand_offsets, k_cache, v_cache, hist_offsets, timestamps,
                    hist_timestamps, pos_bias, time_bias, heads: int, d: int, alpha: float,
                    n: float, dtype: str, tokens, head_ids,
                    lib: Optional[ctypes.CDLL] = None) -> np.ndarray:
    """Sampled candidate rows (m, d) of fwd_rab_cached."""
    lib = lib or load()
    q, k, v, kc, vc, coff, hoff, ts, hts, wp, wt = _rab_cached_args(
            q, k, v, k_cache, v_cache, cand_offsets, hist_offsets, timestamps, hist_timestamps,
            pos_bias, time_bias, heads, d, dtype)
    tok = np.ascontiguousarray(tokens, dtype=np.int64)
    hd = np.ascontiguousarray(head_ids, dtype=np.int32)
    if tok.shape != hd.shape:
        raise ValueError("tokens and head_ids differ in length")
    out = np.zeros((len(tok), d), dtype=np.float64)
    rc = lib.hstu_oracle_rows_rab_cached(_ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc),
                                         _DTYPE_CODE[dtype], _ptr(coff), _ptr(hoff), _ptr(ts),
                                         _ptr(hts), _ptr(wp), len(wp), _ptr(wt), len(wt),
                                         len(coff) - 1, heads, d, float(alpha), float(n),
                                         _ptr(tok), _ptr(hd), len(tok), _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the sampled rows")
    return out


def fwd_rab(q, k, v, offsets, timestamps, pos_bias, time_bias, heads: int, d: int,
            alpha: float, n: float, dtype: str, lib: Optional[ctypes.CDLL] = None,
            num_targets=None) -> np.ndarray:
    """Full fp64 output (T, heads, d) of the causal forward with the relative
    attention bias (target-aware mask and candidate positions when
    num_targets is given); pos_bias / time_bias are given as the float32
    values the GPU call gets (widened exactly)."""
    lib = lib or load()
    q, k, v, off, ts, wp, wt = _rab_args(q, k, v, offsets, timestamps, pos_bias, time_bias,
                                         heads, d, dtype)
    tg = _targets(num_targets, len(off) - 1)
    out = np.zeros((int(off[-1]) if len(off) else 0, heads, d), dtype=np.float64)
    rc = lib.hstu_oracle_fwd_rab_targets(_ptr(q), _ptr(k), _ptr(v), _DTYPE_CODE[dtype],
                                         _ptr(off), None if tg is None else _ptr(tg), _ptr(ts),
                                         _ptr(wp), len(wp), _ptr(wt), len(wt), len(off) - 1,
                                         heads, d, float(alpha), float(n), _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (malformed offsets or sizes)")
    return out


def rows_rab(q, k, v, offsets, timestamps, pos_bias, time_bias, heads: int, d: int,
             alpha: float, n: float, dtype: str, tokens, head_ids,
             lib: Optional[ctypes.CDLL] = None, num_targets=None) -> np.ndarray:
    """fp64 outputs (m, d) at global tokens[m], heads head_ids[m], of the same."""
    lib = lib or load()
    q, k, v, off, ts, wp, wt = _rab_args(q, k, v, offsets, timestamps, pos_bias, time_bias,
                                         heads, d, dtype)
    tg = _targets(num_targets, len(off) - 1)
    tok = np.ascontiguousarray(tokens, dtype=np.int64)
    hd = np.ascontiguousarray(head_ids, dtype=np.int32)
    if tok.shape != hd.shape:
        raise ValueError("tokens and head_ids differ in length")
    out = np.zeros((len(tok), d), dtype=np.float64)
    rc = lib.hstu_oracle_rows_rab_targets(_ptr(q), _ptr(k), _ptr(v), _DTYPE_CODE[dtype],
                                          _ptr(off), None if tg is None else _ptr(tg), _ptr(ts),
                                          _ptr(wp), len(wp), _ptr(wt), len(wt), len(off) - 1,
                                          heads, d, float(alpha), float(n), _ptr(tok), _ptr(hd),
                                          len(tok), _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the sampled rows")
    return out


def bwd_rab(q, k, v, dout, offsets, timestamps, pos_bias, time_bias, heads: int, d: int,
            alpha: float, n: float, dtype: str, lib: Optional[ctypes.CDLL] = None,
            num_targets=None):
    """(dq, dk, dv, dpos, dtime): fp64 gradients of fwd_rab (with num_targets:
    of its target-aware form) for upstream gradient dout; dq/dk/dv
    (T, heads, d), dpos [npos], dtime [ntime]."""
    lib = lib or load()
    q, k, v, off, ts, wp, wt = _rab_args(q, k, v, offsets, timestamps, pos_bias, time_bias,
                                         heads, d, dtype)
    tg = _targets(num_targets, len(off) - 1)
    dout = _storage(dout, dtype)
    T = int(off[-1]) if len(off) else 0
    if dout.size < T * heads * d:
        raise ValueError("dout smaller than offsets imply")
    dq, dk, dv = (np.zeros((T, heads, d), dtype=np.float64) for _ in range(3))
    dpos, dtime = np.zeros(len(wp)), np.zeros(len(wt))
    rc = lib.hstu_oracle_bwd_rab_targets(_ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                         _DTYPE_CODE[dtype], _ptr(off),
                                         None if tg is None else _ptr(tg), _ptr(ts), _ptr(wp),
                                         len(wp), _ptr(wt), len(wt), len(off) - 1, heads, d,
                                         float(alpha), float(n), _ptr(dq), _ptr(dk), _ptr(dv),
                                         _ptr(dpos), _ptr(dtime))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (malformed offsets or sizes)")
    return dq, dk, dv, dpos, dtime


BWD_KIND = {"dq": 0, "dk": 1, "dv": 2}


def bwd_rab_rows(q, k, v, dout, offsets, timestamps, pos_bias, time_bias, heads: int, d: int,
                 alpha: float, n: float, dtype: str, kind: str, tokens, head_ids,
                 lib: Optional[ctypes.CDLL] = None, num_targets=None) -> np.ndarray:
    """Sampled rows (m, d) of dq (at query tokens), dk or dv (at key tokens)
    of bwd_rab."""
    lib = lib or load()
    q, k, v, off, ts, wp, wt = _rab_args(q, k, v, offsets, timestamps, pos_bias, time_bias,
                                         heads, d, dtype)
    tg = _targets(num_targets, len(off) - 1)
    dout = _storage(dout, dtype)
    tok = np.ascontiguousarray(tokens, dtype=np.int64)
    hd = np.ascontiguousarray(head_ids, dtype=np.int32)
    if tok.shape != hd.shape:
        raise ValueError("tokens and head_ids differ in length")
    out = np.zeros((len(tok), d), dtype=np.float64)
    rc = lib.hstu_oracle_bwd_rab_rows_targets(_ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                              _DTYPE_CODE[dtype], _ptr(off),
                                              None if tg is None else _ptr(tg), _ptr(ts),
                                              _ptr(wp), len(wp), _ptr(wt), len(wt), len(off) - 1,
                                              heads, d, float(alpha), float(n), BWD_KIND[kind],
                                              _ptr(tok), _ptr(hd), len(tok), _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the sampled rows")
    return out


def bwd_rows(q, k, v, dout, offsets, heads: int, d: int, alpha: float, n: float, dtype: str,
             kind: str, tokens, head_ids, lib: Optional[ctypes.CDLL] = None,
             num_targets=None) -> np.ndarray:
    """fp64 gradient rows (m, d): kind 'dq' at query tokens[m], 'dk' / 'dv' at
    key tokens[m], heads head_ids[m]."""
    lib = lib or load()
    q, k, v, dout = (_storage(a, dtype) for a in (q, k, v, dout))
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    tg = _targets(num_targets, len(off) - 1)
    tok = np.ascontiguousarray(tokens, dtype=np.int64)
    hd = np.ascontiguousarray(head_ids, dtype=np.int32)
    if tok.shape != hd.shape:
        raise ValueError("tokens and head_ids differ in length")
    out = np.zeros((len(tok), d), dtype=np.float64)
    rc = lib.hstu_oracle_bwd_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _DTYPE_CODE[dtype],
                                  _ptr(off), None if tg is None else _ptr(tg), len(off) - 1,
                                  heads, d, float(alpha), float(n), BWD_KIND[kind], _ptr(tok),
                                  _ptr(hd), len(tok), _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the sampled rows")
    return out


def _f64(a, n: int) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float64)
    if a.shape != (n,):
        raise ValueError(f"expected {n} parameters, got shape {a.shape}")
    return a


def layer_in(x, w1, b1, heads: int, d: int, dtype: str, lib: Optional[ctypes.CDLL] = None):
    """(u, v, q, k), each fp64 (T, heads, d): silu(x W1^T + b1) split in that
    order.  x: (T, d_model), w1: (4 heads d, d_model) in the storage type."""
    lib = lib or load()
    x, w1 = _storage(x, dtype), _storage(w1, dtype)
    T, dm = x.shape
    hd = heads * d
    if w1.shape != (4 * hd, dm):
        raise ValueError("w1 must be (4 * heads * d, d_model)")
    b1 = _f64(b1, 4 * hd)
    outs = [np.zeros((T, heads, d), dtype=np.float64) for _ in range(4)]
    rc = lib.hstu_oracle_layer_in(_ptr(x), _ptr(w1), _ptr(b1), _DTYPE_CODE[dtype], T, dm, heads,
                                  d, *(_ptr(o) for o in outs))
    if rc != 0:
        raise ValueError("oracle rejected the layer arguments")
    return tuple(outs)


def layer_out(attn, u, x, gamma, beta, eps: float, w2, b2, heads: int, d: int, dtype: str,
              lib: Optional[ctypes.CDLL] = None) -> np.ndarray:
    """y fp64 (T, d_model) = x + (LN(attn) * u) W2^T + b2.  attn, u: (T, heads,
    d); x: (T, d_model); w2: (d_model, heads d), all in the storage type."""
    lib = lib or load()
    attn, u, x, w2 = (_storage(a, dtype) for a in (attn, u, x, w2))
    T, dm = x.shape
    hd = heads * d
    if attn.size != T * hd or u.size != T * hd or w2.shape != (dm, hd):
        raise ValueError("layer_out shapes do not match")
    gamma, beta, b2 = _f64(gamma, hd), _f64(beta, hd), _f64(b2, dm)
    y = np.zeros((T, dm), dtype=np.float64)
    rc = lib.hstu_oracle_layer_out(_ptr(attn), _ptr(u), _ptr(x), _ptr(gamma), _ptr(beta),
                                   float(eps), _ptr(w2), _ptr(b2), _DTYPE_CODE[dtype], T, dm,
                                   heads, d, _ptr(y))
    if rc != 0:
        raise ValueError("oracle rejected the layer arguments")
    return y


def threads(lib: Optional[ctypes.CDLL] = None) -> int:
    return int((lib or load()).hstu_oracle_threads())


# ---------------------------------------------------------------------------
# Dense pair-set evaluation (numpy fp64), for small inputs.
# ---------------------------------------------------------------------------

def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 image of stored values (bf16 bits are widened through fp32)."""
    if dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    return np.asarray(x).astype(np.float64)


def _silu(x: np.ndarray) -> np.ndarray:
    # x * sigmoid(x); np.exp(-|x|) never overflows.
    e = np.exp(-np.abs(x))
    sig = np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return x * sig


def sees(s: int, t: int = 0) -> np.ndarray:
    """Boolean (s, s) matrix: entry (row, key) is True iff the row sees the
    key.  Causal: key <= row.  With t candidates (HSTU paper translation,
    Appendix H, Algorithm 1), rows and keys past the history h = s - t also
    need key < h or key == row."""
    r = np.arange(s)[:, None]
    c = np.arange(s)[None, :]
    h = s - t
    return (c <= r) & ((c < h) | (c == r))


def dense_pairs(q, k, v, offsets, heads: int, d: int, alpha: float, n: float,
                dtype: str, num_targets=None) -> np.ndarray:
    """out[r, h] = (1/n) * sum over keys c that row r sees of
    silu(alpha * <q[r, h], k[c, h]>) * v[c, h], per sequence, every
    (row, key) pair's score formed with einsum and pairs the row does not see
    left out of the sum (their weight is set to zero before the sum over keys).
    The visibility is ``sees`` (causal, or target-aware with the sequence's
    candidate count)."""
    Q, K, V = (widen(a, dtype).reshape(-1, heads, d) for a in (q, k, v))
    off = np.asarray(offsets, dtype=np.int64)
    out = np.zeros((int(off[-1]), heads, d), dtype=np.float64)
    for i in range(len(off) - 1):
        a, b = int(off[i]), int(off[i + 1])
        s = b - a
        if s == 0:
            continue
        t = 0 if num_targets is None else min(max(int(num_targets[i]), 0), s)
        seen = sees(s, t)
        score = np.einsum("rhe,che->hrc", Q[a:b], K[a:b])
        w = np.where(seen[None, :, :], _silu(alpha * score), 0.0)
        out[a:b] = np.einsum("hrc,che->rhe", w, V[a:b]) / n
    return out