"""HSTU jagged causal attention forward on AMD MI355X (gfx950).

A thin ctypes binding over ``libhstu.so`` (the C ABI in ``include/hstu.h``).
Every step of the computation runs in the library's HIP kernels; this module
only checks and marshals arguments.  PyTorch supplies device memory and the
current stream.  There is no CPU fallback: without the built library every
call raises.

    out = hstu_attn_fwd(q, k, v, seq_offsets, alpha, n)

q, k, v: (T, heads, d) CUDA tensors (bfloat16, float16 or float32), contiguous;
seq_offsets: int32 CUDA tensor [num_seqs + 1] of prefix sums.

Also: hstu_attn_fwd_{bf16,fp16,fp32} (type fixed), hstu_attn_fwd_targets
(target-aware mask), hstu_attn_fwd_rab / hstu_attn_bwd_rab (relative
attention bias), hstu_attn_fwd_rab_targets / hstu_attn_bwd_rab_targets (the
bias under the target-aware mask),
hstu_attn_fwd_cached (candidates against a cached history),
hstu_attn_fwd_dense / hstu_attn_bwd_dense ((B, heads, S, d) tensors),
hstu_attn_bwd (dq, dk, dv), hstu_layer_in_proj /
hstu_layer_out_proj (the layer's projections), hstu_attn_fwd_noalloc (the
forward with no allocation in the library), and the utilities
hstu_validate_offsets, hstu_release_workspace, hstu_profile_enable/read.
The offsets live on the device and are not read by the host: keeping them
consistent with the tensors' lengths is the caller's part (see
hstu_validate_offsets).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libhstu.so")

HSTU_OK = 0
HSTU_ERR_INVALID_ARG = -1
HSTU_ERR_UNSUPPORTED = -2
HSTU_ERR_HIP = -3
HSTU_ERR_NO_MEMORY = -4
HSTU_ERR_BAD_OFFSETS = -5
HSTU_ERR_SCRATCH_LIMIT = -6
HSTU_NOALLOC_SCRATCH_BYTES = 1 << 20

HSTU_BF16, HSTU_FP16, HSTU_FP32 = 0, 1, 2

# Every symbol include/hstu.h declares.
EXPORTS = ("hstu_attn_fwd", "hstu_attn_fwd_bf16", "hstu_attn_fwd_fp16", "hstu_attn_fwd_fp32",
           "hstu_attn_fwd_targets", "hstu_attn_fwd_cached", "hstu_attn_fwd_dense",
           "hstu_attn_fwd_rab", "hstu_attn_fwd_rab_targets", "hstu_attn_bwd_rab", "hstu_attn_bwd",
           "hstu_attn_bwd_dense", "hstu_layer_in_proj", "hstu_layer_out_proj",
           "hstu_attn_bwd_targets", "hstu_validate_offsets", "hstu_status_string", "hstu_last_hip_error",
           "hstu_release_workspace", "hstu_profile_enable", "hstu_profile_read",
           "hstu_attn_fwd_noalloc", "hstu_attn_bwd_rab_targets", "hstu_attn_fwd_rab_cached")


class HstuError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(what)


class KernelTimes(ctypes.Structure):
    _fields_ = [("calls", ctypes.c_int64), ("sched_ms", ctypes.c_double),
                ("attn_ms", ctypes.c_double), ("dropped", ctypes.c_int64),
                ("attn_min_ms", ctypes.c_double), ("attn_median_ms", ctypes.c_double),
                ("clock_mhz", ctypes.c_double)]


_lib: Optional[ctypes.CDLL] = None


def library_path() -> str:
    return LIBRARY


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libhstu.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIBRARY
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is missing: build it with "
            "`python -m generative_recommendation_attention_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(p)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    fwd = [vp, vp, vp, vp, i32, i32, i32, f32, f32, vp, vp]
    lib.hstu_attn_fwd.argtypes = fwd + [ctypes.c_int]
    lib.hstu_attn_fwd.restype = ctypes.c_int
    lib.hstu_attn_fwd_noalloc.argtypes = fwd + [ctypes.c_int]
    lib.hstu_attn_fwd_noalloc.restype = ctypes.c_int
    for name in ("hstu_attn_fwd_bf16", "hstu_attn_fwd_fp16", "hstu_attn_fwd_fp32"):
        getattr(lib, name).argtypes = fwd
        getattr(lib, name).restype = ctypes.c_int
    lib.hstu_attn_fwd_targets.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, f32, f32, vp, vp,
                                          ctypes.c_int]
    lib.hstu_attn_fwd_targets.restype = ctypes.c_int
    lib.hstu_attn_fwd_cached.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, f32, f32, vp,
                                         vp, ctypes.c_int]
    lib.hstu_attn_fwd_cached.restype = ctypes.c_int
    lib.hstu_attn_fwd_dense.argtypes = [vp, vp, vp, i32, i32, i32, i32, f32, f32, vp, vp,
                                        ctypes.c_int]
    lib.hstu_attn_fwd_dense.restype = ctypes.c_int
    lib.hstu_attn_fwd_rab.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, f32,
                                      f32, vp, vp, ctypes.c_int]
    lib.hstu_attn_fwd_rab.restype = ctypes.c_int
    lib.hstu_attn_fwd_rab_targets.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32,
                                              i32, f32, f32, vp, vp, ctypes.c_int]
    lib.hstu_attn_fwd_rab_targets.restype = ctypes.c_int
    lib.hstu_attn_fwd_rab_cached.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i32,
                                             i32, i32, i32, f32, f32, vp, vp, ctypes.c_int]
    lib.hstu_attn_fwd_rab_cached.restype = ctypes.c_int
    lib.hstu_attn_bwd_rab.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, f32,
                                      f32, vp, vp, vp, vp, vp, vp, ctypes.c_int]
    lib.hstu_attn_bwd_rab.restype = ctypes.c_int
    lib.hstu_attn_bwd_rab_targets.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32,
                                              i32, i32, f32, f32, vp, vp, vp, vp, vp, vp,
                                              ctypes.c_int]
    lib.hstu_attn_bwd_rab_targets.restype = ctypes.c_int
    i64 = ctypes.c_int64
    lib.hstu_layer_in_proj.argtypes = [vp, vp, vp, i64, i32, i32, i32, vp, vp, vp, vp, vp,
                                       ctypes.c_int]
    lib.hstu_layer_in_proj.restype = ctypes.c_int
    lib.hstu_layer_out_proj.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, i64, i32, i32, i32, vp,
                                        vp, ctypes.c_int]
    lib.hstu_layer_out_proj.restype = ctypes.c_int
    lib.hstu_attn_bwd_dense.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, f32, f32, vp, vp, vp,
                                        vp, ctypes.c_int]
    lib.hstu_attn_bwd_dense.restype = ctypes.c_int
    lib.hstu_attn_bwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, f32, f32, vp, vp, vp, vp,
                                  ctypes.c_int]
    lib.hstu_attn_bwd.restype = ctypes.c_int
    lib.hstu_attn_bwd_targets.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, f32, f32, vp, vp,
                                          vp, vp, ctypes.c_int]
    lib.hstu_attn_bwd_targets.restype = ctypes.c_int
    lib.hstu_validate_offsets.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_int64), vp]
    lib.hstu_validate_offsets.restype = ctypes.c_int
    lib.hstu_status_string.argtypes = [ctypes.c_int]
    lib.hstu_status_string.restype = ctypes.c_char_p
    lib.hstu_last_hip_error.argtypes = []
    lib.hstu_last_hip_error.restype = ctypes.c_int
    lib.hstu_release_workspace.argtypes = []
    lib.hstu_release_workspace.restype = None
    lib.hstu_profile_enable.argtypes = [ctypes.c_int]
    lib.hstu_profile_enable.restype = ctypes.c_int
    lib.hstu_profile_read.argtypes = [ctypes.POINTER(KernelTimes), ctypes.c_int]
    lib.hstu_profile_read.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _check(status: int, what: str) -> None:
    if status != HSTU_OK:
        lib = load_library()
        msg = lib.hstu_status_string(status).decode()
        if status == HSTU_ERR_HIP:
            msg += f" (hipError {lib.hstu_last_hip_error()})"
        raise HstuError(status, f"{what}: {msg}")


def _dtype_code(t) -> int:
    import torch
    codes = {torch.bfloat16: HSTU_BF16, torch.float16: HSTU_FP16, torch.float32: HSTU_FP32}
    if t.dtype not in codes:
        raise TypeError(f"unsupported element type {t.dtype}")
    return codes[t.dtype]


def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _check_tensors(q, k, v, seq_offsets, out):
    import torch
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one (T, heads, d) shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one element type")
    for t in (q, k, v, seq_offsets):
        if not t.is_cuda:
            raise ValueError("all tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if seq_offsets.dtype != torch.int32 or seq_offsets.dim() != 1 or seq_offsets.numel() < 1:
        raise ValueError("seq_offsets must be a 1-D int32 tensor of num_seqs + 1 entries")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    return out


def hstu_attn_fwd(q, k, v, seq_offsets, alpha: float, n: float, out=None, stream=None):
    """Jagged causal HSTU attention forward; returns `out` (T, heads, d)."""
    out = _check_tensors(q, k, v, seq_offsets, out)
    T, heads, d = q.shape
    num_seqs = seq_offsets.numel() - 1
    lib = load_library()
    st = lib.hstu_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), seq_offsets.data_ptr(),
                           num_seqs, heads, d, float(alpha), float(n), out.data_ptr(),
                           _stream_handle(stream), _dtype_code(q))
    _check(st, "hstu_attn_fwd")
    return out


def hstu_attn_fwd_noalloc(q, k, v, seq_offsets, alpha: float, n: float, out=None, stream=None):
    """hstu_attn_fwd through the library's allocation-free entry point (its
    work list in a fixed per-GPU device array; see include/hstu.h).  The
    library allocates nothing; `out` is allocated here with torch if not
    given."""
    out = _check_tensors(q, k, v, seq_offsets, out)
    T, heads, d = q.shape
    num_seqs = seq_offsets.numel() - 1
    lib = load_library()
    st = lib.hstu_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                   seq_offsets.data_ptr(), num_seqs, heads, d, float(alpha),
                                   float(n), out.data_ptr(), _stream_handle(stream),
                                   _dtype_code(q))
    _check(st, "hstu_attn_fwd_noalloc")
    return out


def hstu_attn_fwd_rab(q, k, v, seq_offsets, timestamps, pos_bias, time_bias, alpha: float,
                      n: float, out=None, stream=None):
    """Jagged causal HSTU attention forward with the relative attention bias
    rab(r, c) = pos_bias[r - c] + time_bias[min(floor(log2(ts_r - ts_c + 1)),
    len(time_bias) - 1)] added to alpha * <q_r, k_c> before SiLU.
    timestamps: int32 GPU tensor of T entries; pos_bias, time_bias: float32
    GPU tensors (the time table holds 1 to 32 entries)."""
    out = _check_tensors(q, k, v, seq_offsets, out)
    T, heads, d = q.shape
    _check_rab(T, timestamps, pos_bias, time_bias)
    num_seqs = seq_offsets.numel() - 1
    lib = load_library()
    st = lib.hstu_attn_fwd_rab(q.data_ptr(), k.data_ptr(), v.data_ptr(), seq_offsets.data_ptr(),
                               timestamps.data_ptr(), pos_bias.data_ptr(), pos_bias.numel(),
                               time_bias.data_ptr(), time_bias.numel(), num_seqs, heads, d,
                               float(alpha), float(n), out.data_ptr(), _stream_handle(stream),
                               _dtype_code(q))
    _check(st, "hstu_attn_fwd_rab")
    return out


def _check_rab(T, timestamps, pos_bias, time_bias):
    import torch
    if (timestamps.dtype != torch.int32 or timestamps.shape != (T,) or not timestamps.is_cuda or
            not timestamps.is_contiguous()):
        raise ValueError("timestamps must be a contiguous int32 GPU tensor of T entries")
    for name, t in (("pos_bias", pos_bias), ("time_bias", time_bias)):
        if t.dtype != torch.float32 or t.dim() != 1 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 1-D float32 GPU tensor")


def _check_targets(num_targets, num_seqs):
    import torch
    if (num_targets.dtype != torch.int32 or num_targets.dim() != 1 or
            num_targets.numel() != num_seqs or not num_targets.is_cuda or
            not num_targets.is_contiguous()):
        raise ValueError("num_targets must be a contiguous 1-D int32 GPU tensor of num_seqs entries")


def hstu_attn_fwd_rab_targets(q, k, v, seq_offsets, num_targets, timestamps, pos_bias, time_bias,
                              alpha: float, n: float, out=None, stream=None):
    """hstu_attn_fwd_rab under the target-aware mask of hstu_attn_fwd_targets
    (M-FALCON): a candidate row takes the position right after its sequence's
    history (distance hist - c to history key c, 0 to itself) and keeps its
    own timestamp, so each candidate's output is that of the history followed
    by that candidate alone."""
    out = _check_tensors(q, k, v, seq_offsets, out)
    T, heads, d = q.shape
    num_seqs = seq_offsets.numel() - 1
    _check_targets(num_targets, num_seqs)
    _check_rab(T, timestamps, pos_bias, time_bias)
    lib = load_library()
    st = lib.hstu_attn_fwd_rab_targets(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                       seq_offsets.data_ptr(), num_targets.data_ptr(),
                                       timestamps.data_ptr(), pos_bias.data_ptr(),
                                       pos_bias.numel(), time_bias.data_ptr(), time_bias.numel(),
                                       num_seqs, heads, d, float(alpha), float(n), out.data_ptr(),
                                       _stream_handle(stream), _dtype_code(q))
    _check(st, "hstu_attn_fwd_rab_targets")
    return out


def hstu_attn_fwd_targets(q, k, v, seq_offsets, num_targets, alpha: float, n: float, out=None,
                          stream=None):
    """HSTU attention forward under the target-aware mask: the last
    num_targets[i] tokens of sequence i are candidates that see the history
    and themselves only.  num_targets: int32 device tensor of num_seqs entries."""
    out = _check_tensors(q, k, v, seq_offsets, out)
    num_seqs = seq_offsets.numel() - 1
    _check_targets(num_targets, num_seqs)
    T, heads, d = q.shape
    lib = load_library()
    st = lib.hstu_attn_fwd_targets(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                   seq_offsets.data_ptr(), num_targets.data_ptr(), num_seqs,
                                   heads, d, float(alpha), float(n), out.data_ptr(),
                                   _stream_handle(stream), _dtype_code(q))
    _check(st, "hstu_attn_fwd_targets")
    return out


def _check_cache(q, k_cache, v_cache, hist_offsets, num_seqs):
    import torch
    for t in (k_cache, v_cache):
        if (t.dim() != 3 or t.shape[1:] != q.shape[1:] or t.dtype != q.dtype or not t.is_cuda
                or not t.is_contiguous()):
            raise ValueError("k_cache and v_cache must be contiguous GPU tensors "
                             "(T_hist, heads, d) of q's element type")
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share one shape")
    if (hist_offsets.dtype != torch.int32 or hist_offsets.dim() != 1 or
            hist_offsets.numel() != num_seqs + 1 or not hist_offsets.is_cuda or
            not hist_offsets.is_contiguous()):
        raise ValueError("hist_offsets must be a contiguous 1-D int32 GPU tensor of "
                         "num_seqs + 1 entries")


def hstu_attn_fwd_cached(q, k, v, cand_offsets, k_cache, v_cache, hist_offsets, alpha: float,
                         n: float, out=None, stream=None):
    """Candidates (q, k, v: (T_cand, heads, d), offsets cand_offsets) scored
    against a cached history (k_cache, v_cache: (T_hist, heads, d), offsets
    hist_offsets): each candidate sees its request's history and itself."""
    out = _check_tensors(q, k, v, cand_offsets, out)
    num_seqs = cand_offsets.numel() - 1
    T, heads, d = q.shape
    _check_cache(q, k_cache, v_cache, hist_offsets, num_seqs)
    lib = load_library()
    if T == 0:
        return out   # no candidate rows: nothing to compute
    empty_cache = k_cache.numel() == 0   # no history at all: the library takes null caches
    st = lib.hstu_attn_fwd_cached(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  cand_offsets.data_ptr(),
                                  None if empty_cache else k_cache.data_ptr(),
                                  None if empty_cache else v_cache.data_ptr(),
                                  hist_offsets.data_ptr(), num_seqs, heads,
                                  d, float(alpha), float(n), out.data_ptr(),
                                  _stream_handle(stream), _dtype_code(q))
    _check(st, "hstu_attn_fwd_cached")
    return out


def hstu_attn_fwd_rab_cached(q, k, v, cand_offsets, k_cache, v_cache, hist_offsets, timestamps,
                             hist_timestamps, pos_bias, time_bias, alpha: float, n: float,
                             out=None, stream=None):
    """hstu_attn_fwd_cached with the relative attention bias: a candidate sits
    right after its request's cached history (distance h - c to history row c,
    0 to itself) and keeps its own timestamp.  timestamps: int32 GPU tensor of
    T_cand entries; hist_timestamps: int32 GPU tensor of T_hist entries (the
    layout of k_cache); pos_bias, time_bias as in hstu_attn_fwd_rab."""
    import torch
    out = _check_tensors(q, k, v, cand_offsets, out)
    num_seqs = cand_offsets.numel() - 1
    T, heads, d = q.shape
    _check_cache(q, k_cache, v_cache, hist_offsets, num_seqs)
    _check_rab(T, timestamps, pos_bias, time_bias)
    if (hist_timestamps.dtype != torch.int32 or hist_timestamps.shape != (k_cache.shape[0],) or
            not hist_timestamps.is_cuda or not hist_timestamps.is_contiguous()):
        raise ValueError("hist_timestamps must be a contiguous int32 GPU tensor of T_hist entries")
    lib = load_library()
    if T == 0:
        return out
    empty_cache = k_cache.numel() == 0
    st = lib.hstu_attn_fwd_rab_cached(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                      cand_offsets.data_ptr(),
                                      None if empty_cache else k_cache.data_ptr(),
                                      None if empty_cache else v_cache.data_ptr(),
                                      hist_offsets.data_ptr(), timestamps.data_ptr(),
                                      None if empty_cache else hist_timestamps.data_ptr(),
                                      pos_bias.data_ptr(), pos_bias.numel(), time_bias.data_ptr(),
                                      time_bias.numel(), num_seqs, heads, d, float(alpha),
                                      float(n), out.data_ptr(), _stream_handle(stream),
                                      _dtype_code(q))
    _check(st, "hstu_attn_fwd_rab_cached")
    return out


def _typed(name: str, code: int):
    def fn(q, k, v, seq_offsets, alpha: float, n: float, out=None, stream=None):
        if _dtype_code(q) != code:
            raise TypeError(f"{name} takes {['bfloat16', 'float16', 'float32'][code]} tensors")
        out = _check_tensors(q, k, v, seq_offsets, out)
        T, heads, d = q.shape
        lib = load_library()
        st = getattr(lib, name)(q.data_ptr(), k.data_ptr(), v.data_ptr(), seq_offsets.data_ptr(),
                                seq_offsets.numel() - 1, heads, d, float(alpha), float(n),
                                out.data_ptr(), _stream_handle(stream))
        _check(st, name)
        return out
    fn.__name__ = name
    fn.__doc__ = f"{name}: hstu_attn_fwd with the element type fixed."
    return fn


hstu_attn_fwd_bf16 = _typed("hstu_attn_fwd_bf16", HSTU_BF16)
hstu_attn_fwd_fp16 = _typed("hstu_attn_fwd_fp16", HSTU_FP16)
hstu_attn_fwd_fp32 = _typed("hstu_attn_fwd_fp32", HSTU_FP32)


def hstu_validate_offsets(seq_offsets, stream=None) -> int:
    """Synchronous device-offset check; returns T = off[num_seqs]."""
    lib = load_library()
    total = ctypes.c_int64(0)
    st = lib.hstu_validate_offsets(seq_offsets.data_ptr(), seq_offsets.numel() - 1,
                                   ctypes.byref(total), _stream_handle(stream))
    _check(st, "hstu_validate_offsets")
    return int(total.value)


def hstu_release_workspace() -> None:
    load_library().hstu_release_workspace()


def hstu_profile_enable(on: bool) -> None:
    _check(load_library().hstu_profile_enable(1 if on else 0), "hstu_profile_enable")


def hstu_profile_read(reset: bool = True) -> KernelTimes:
    t = KernelTimes()
    _check(load_library().hstu_profile_read(ctypes.byref(t), 1 if reset else 0),
           "hstu_profile_read")
    return t


def hstu_attn_bwd(q, k, v, dout, seq_offsets, alpha: float, n: float, num_targets=None,
                  grads=None, stream=None):
    """Gradients (dq, dk, dv) of the forward (target-aware when num_targets is
    given) for the upstream gradient dout.  `grads` may supply three
    preallocated output tensors."""
    import torch
    _check_tensors(q, k, v, seq_offsets, torch.empty_like(q))
    if dout.shape != q.shape or dout.dtype != q.dtype or not dout.is_cuda or \
            not dout.is_contiguous():
        raise ValueError("dout must be a contiguous GPU tensor shaped and typed like q")
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q))
    for t in grads:
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("gradient outputs must be contiguous GPU tensors shaped like q")
    dq, dk, dv = grads
    T, heads, d = q.shape
    num_seqs = seq_offsets.numel() - 1
    if T == 0:
        return dq, dk, dv
    lib = load_library()
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), seq_offsets.data_ptr())
    tail = (num_seqs, heads, d, float(alpha), float(n), dq.data_ptr(), dk.data_ptr(),
            dv.data_ptr(), _stream_handle(stream), _dtype_code(q))
    if num_targets is None:
        st = lib.hstu_attn_bwd(*args, *tail)
        _check(st, "hstu_attn_bwd")
    else:
        if (num_targets.dtype != torch.int32 or num_targets.dim() != 1 or
                num_targets.numel() != num_seqs or not num_targets.is_cuda or
                not num_targets.is_contiguous()):
            raise ValueError("num_targets must be a contiguous 1-D int32 GPU tensor of "
                             "num_seqs entries")
        st = lib.hstu_attn_bwd_targets(*args, num_targets.data_ptr(), *tail)
        _check(st, "hstu_attn_bwd_targets")
    return dq, dk, dv


def hstu_attn_bwd_rab(q, k, v, dout, seq_offsets, timestamps, pos_bias, time_bias,
                      alpha: float, n: float, grads=None, stream=None):
    """Gradients of hstu_attn_fwd_rab for the upstream gradient dout:
    (dq, dk, dv, d_pos_bias, d_time_bias), the last two float32 like the
    tables.  `grads` may supply the five output tensors."""
    return _bwd_rab(q, k, v, dout, seq_offsets, None, timestamps, pos_bias, time_bias, alpha, n,
                    grads, stream)


def hstu_attn_bwd_rab_targets(q, k, v, dout, seq_offsets, num_targets, timestamps, pos_bias,
                              time_bias, alpha: float, n: float, grads=None, stream=None):
    """Gradients of hstu_attn_fwd_rab_targets (num_targets: int32 [num_seqs]),
    returned as in hstu_attn_bwd_rab."""
    return _bwd_rab(q, k, v, dout, seq_offsets, num_targets, timestamps, pos_bias, time_bias,
                    alpha, n, grads, stream)


def _bwd_rab(q, k, v, dout, seq_offsets, num_targets, timestamps, pos_bias, time_bias,
             alpha: float, n: float, grads, stream):
    import torch
    _check_tensors(q, k, v, seq_offsets, torch.empty_like(q))
    T, heads, d = q.shape
    num_seqs = seq_offsets.numel() - 1
    if dout.shape != q.shape or dout.dtype != q.dtype or not dout.is_cuda or \
            not dout.is_contiguous():
        raise ValueError("dout must be a contiguous GPU tensor shaped and typed like q")
    _check_rab(T, timestamps, pos_bias, time_bias)
    if num_targets is not None:
        _check_targets(num_targets, num_seqs)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q),
                 torch.empty_like(pos_bias), torch.empty_like(time_bias))
    dq, dk, dv, dpos, dtime = grads
    for t in (dq, dk, dv):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("gradient outputs must be contiguous GPU tensors shaped like q")
    for t, ref in ((dpos, pos_bias), (dtime, time_bias)):
        if t.shape != ref.shape or t.dtype != torch.float32 or not t.is_contiguous() or \
                not t.is_cuda:
            raise ValueError("table gradients must be contiguous float32 GPU tensors shaped "
                             "like the tables")
    if T == 0:
        dpos.zero_()
        dtime.zero_()
        return dq, dk, dv, dpos, dtime
    lib = load_library()
    head = (q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), seq_offsets.data_ptr())
    tail = (timestamps.data_ptr(), pos_bias.data_ptr(), pos_bias.numel(), time_bias.data_ptr(),
            time_bias.numel(), num_seqs, heads, d, float(alpha), float(n), dq.data_ptr(),
            dk.data_ptr(), dv.data_ptr(), dpos.data_ptr(), dtime.data_ptr(),
            _stream_handle(stream), _dtype_code(q))
    if num_targets is None:
        _check(lib.hstu_attn_bwd_rab(*head, *tail), "hstu_attn_bwd_rab")
    else:
        _check(lib.hstu_attn_bwd_rab_targets(*head, num_targets.data_ptr(), *tail),
               "hstu_attn_bwd_rab_targets")
    return dq, dk, dv, dpos, dtime


def hstu_attn_fwd_dense(q, k, v, alpha: float, n: float, out=None, stream=None):
    """Causal HSTU attention forward on dense (batch, heads, seq_len, d)
    tensors (every position is a token); returns `out` of the same shape."""
    import torch
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one (batch, heads, seq_len, d) shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one element type")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous GPU tensors")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    B, heads, S, d = q.shape
    if q.numel() == 0:
        return out
    lib = load_library()
    st = lib.hstu_attn_fwd_dense(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, heads, S, d,
                                 float(alpha), float(n), out.data_ptr(), _stream_handle(stream),
                                 _dtype_code(q))
    _check(st, "hstu_attn_fwd_dense")
    return out


def _gpu_contig(name, t, dtype=None, shape=None):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def hstu_layer_in_proj(x, w1, b1, heads: int, d: int, out=None, stream=None):
    """(u, v, q, k) = split(silu(x @ w1.T + b1)), each (T, heads, d).
    x: (T, d_model); w1: (4 heads d, d_model) of x's type; b1: float32."""
    import torch
    T, dm = x.shape
    hd = heads * d
    _gpu_contig("x", x)
    _gpu_contig("w1", w1, x.dtype, (4 * hd, dm))
    _gpu_contig("b1", b1, torch.float32, (4 * hd,))
    if out is None:
        out = tuple(torch.empty((T, heads, d), dtype=x.dtype, device=x.device) for _ in range(4))
    for i, t in enumerate(out):
        _gpu_contig(f"out[{i}]", t, x.dtype, (T, heads, d))
    if T == 0:
        return out
    lib = load_library()
    st = lib.hstu_layer_in_proj(x.data_ptr(), w1.data_ptr(), b1.data_ptr(), T, dm, heads, d,
                                *(t.data_ptr() for t in out), _stream_handle(stream),
                                _dtype_code(x))
    _check(st, "hstu_layer_in_proj")
    return out


def hstu_layer_out_proj(attn, u, x, gamma, beta, eps: float, w2, b2, out=None, stream=None):
    """y = x + (layer_norm(attn) * u) @ w2.T + b2 (norm over heads * d).
    attn, u: (T, heads, d); x: (T, d_model); w2: (d_model, heads d);
    gamma, beta, b2: float32."""
    import torch
    T, heads, d = attn.shape
    hd = heads * d
    dm = x.shape[1]
    _gpu_contig("attn", attn)
    _gpu_contig("u", u, attn.dtype, attn.shape)
    _gpu_contig("x", x, attn.dtype, (T, dm))
    _gpu_contig("w2", w2, attn.dtype, (dm, hd))
    for name, t, n in (("gamma", gamma, hd), ("beta", beta, hd), ("b2", b2, dm)):
        _gpu_contig(name, t, torch.float32, (n,))
    if out is None:
        out = torch.empty_like(x)
    _gpu_contig("out", out, x.dtype, x.shape)
    if T == 0:
        return out
    lib = load_library()
    st = lib.hstu_layer_out_proj(attn.data_ptr(), u.data_ptr(), x.data_ptr(), gamma.data_ptr(),
                                 beta.data_ptr(), float(eps), w2.data_ptr(), b2.data_ptr(), T, dm,
                                 heads, d, out.data_ptr(), _stream_handle(stream),
                                 _dtype_code(attn))
    _check(st, "hstu_layer_out_proj")
    return out


def hstu_attn_bwd_dense(q, k, v, dout, alpha: float, n: float, grads=None, stream=None):
    """Gradients (dq, dk, dv) of hstu_attn_fwd_dense: all tensors
    (batch, heads, seq_len, d)."""
    import torch
    if q.dim() != 4 or any(t.shape != q.shape for t in (k, v, dout)):
        raise ValueError("q, k, v, dout must share one (batch, heads, seq_len, d) shape")
    for t in (q, k, v, dout):
        _gpu_contig("input", t, q.dtype)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q))
    for t in grads:
        _gpu_contig("gradient output", t, q.dtype, q.shape)
    B, heads, S, d = q.shape
    if q.numel() == 0:
        return grads
    lib = load_library()
    dq, dk, dv = grads
    st = lib.hstu_attn_bwd_dense(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), B,
                                 heads, S, d, float(alpha), float(n), dq.data_ptr(),
                                 dk.data_ptr(), dv.data_ptr(), _stream_handle(stream),
                                 _dtype_code(q))
    _check(st, "hstu_attn_bwd_dense")
    return grads
