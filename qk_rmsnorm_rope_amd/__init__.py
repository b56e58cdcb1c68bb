"""Python binding of the qknr C ABI (include/qknr.h): fused QK / KV RMSNorm +
RoPE (+ KV-cache scatter) on AMD MI355X (gfx950).

This module only marshals torch tensors into the ABI's argument structs
(pointers, element strides, dtype codes) and passes torch's current HIP stream.
Every step of both operators runs in the HIP kernels of libqknr.so; there is
no fallback: importing fails loudly if the library has not been built
(``python qk_rmsnorm_rope_amd/_build.py``).

Entry points (same names as the C ABI, without the ``qknr_`` prefix):

* :func:`qk_norm_rope_across_heads` -- across-heads RMSNorm + rotate-half RoPE
  ("Kernel reference: qkv_cte", Design sections 1-2).
* :func:`qk_sumsq_across_heads`, :func:`qk_apply_across_heads` -- the same
  operator split over ranks (step a, then step c with the added sums).
* :func:`qk_norm_rope_per_head` -- the upstream per-head qk-norm + RoPE.
* :func:`interleaved_to_rotate_half` -- the offline lane permutation of an
  interleaved-pair checkpoint (qkv_cte Design section 2).
* :func:`qkv_projection` -- the QKV projection GEMM on matrix cores with the
  across-heads norm's sums of squares in its epilogue (qkv_cte Design section 1).
* :func:`kv_rmsnorm_rope_cache` -- the KvRmsNormRopeCache operator (CANN page,
  formulas 1-5), argument names as on that page's parameter table.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqknr.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python qk_rmsnorm_rope_amd/_build.py, or __graft_entry__.build())")

_lib = ctypes.CDLL(LIB_PATH)

OK, INVALID_ARGUMENT, UNSUPPORTED, DEVICE_ERROR = 0, 1, 2, 3
F32, BF16, F16, INT8, FP8_E4M3FN, FP8_E5M2 = 0, 1, 2, 3, 4, 5
CACHE_NORM, CACHE_PA_BNSD, CACHE_PA_BLK_BNSD = 0, 1, 2
QSHAPE_SCALAR, QSHAPE_CHANNEL, QSHAPE_HEAD_CHANNEL = 0, 1, 2
PROJ_SCALE_ROW, PROJ_SCALE_MX32 = 0, 1

_DTYPE = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16,
          torch.int8: INT8, torch.float8_e4m3fn: FP8_E4M3FN, torch.float8_e5m2: FP8_E5M2}
_CACHE_MODE = {"Norm": CACHE_NORM, "PA": CACHE_PA_BNSD, "PA_BNSD": CACHE_PA_BNSD,
               "PA_BLK_BNSD": CACHE_PA_BLK_BNSD}

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class QkArgs(ctypes.Structure):
    """Mirror of ``qknr_qk_args``."""
    _fields_ = [
        ("dtype", _i32), ("n_q_heads", _i32), ("n_k_heads", _i32), ("head_dim", _i32),
        ("batch", _i64), ("seq", _i64),
        ("q_in", _p), ("k_in", _p), ("q_out", _p), ("k_out", _p),
        ("in_batch_stride", _i64), ("in_token_stride", _i64), ("in_head_stride", _i64),
        ("out_batch_stride", _i64), ("out_token_stride", _i64), ("out_head_stride", _i64),
        ("q_gamma", _p), ("k_gamma", _p), ("cos", _p), ("sin", _p),
        ("rope_batch_stride", _i64), ("rope_token_stride", _i64),
        ("eps", ctypes.c_float), ("apply_norm", _i32), ("apply_rope", _i32), ("sumsq_parts", _i32),
        ("q_norm_channels", _i64), ("k_norm_channels", _i64),
    ]


class ProjArgs(ctypes.Structure):
    """Mirror of ``qknr_proj_args``."""
    _fields_ = [
        ("dtype", _i32), ("scale_mode", _i32), ("rows", _i64), ("in_features", _i64), ("out_features", _i64),
        ("a", _p), ("a_row_stride", _i64), ("w", _p), ("w_row_stride", _i64), ("bias", _p),
        ("out", _p), ("out_row_stride", _i64), ("q_cols", _i64), ("k_cols", _i64), ("sumsq", _p),
        ("a_scale", _p), ("w_scale", _p), ("a_block_scale", _p), ("a_block_scale_stride", _i64),
        ("w_block_scale", _p), ("w_block_scale_stride", _i64),
    ]


class PermuteArgs(ctypes.Structure):
    """Mirror of ``qknr_permute_args``."""
    _fields_ = [
        ("elem_bytes", _i32), ("inverse", _i32), ("outer", _i64), ("axis_len", _i64), ("inner", _i64),
        ("first", _i64), ("n_heads", _i64), ("head_dim", _i64), ("src", _p), ("dst", _p),
    ]


class KvArgs(ctypes.Structure):
    """Mirror of ``qknr_kv_args``."""
    _fields_ = [
        ("dtype", _i32), ("heads", _i32), ("batch", _i64), ("seq", _i64),
        ("kv_dim", _i32), ("rms_size", _i32), ("rope_size", _i32), ("v_dim", _i32),
        ("kv", _p), ("v_optional", _p), ("gamma", _p), ("cos", _p), ("sin", _p),
        ("kv_strides", _i64 * 3), ("v_strides", _i64 * 3), ("rope_strides", _i64 * 3),
        ("index", _p), ("cache_mode", _i32), ("block_size", _i32), ("cache_rows", _i64),
        ("k_cache", _p), ("ckv_cache", _p), ("k_cache_dtype", _i32), ("ckv_cache_dtype", _i32),
        ("k_cache_strides", _i64 * 3), ("ckv_cache_strides", _i64 * 3),
        ("k_scale", _p), ("k_offset", _p), ("v_scale", _p), ("v_offset", _p),
        ("k_qshape", _i32), ("v_qshape", _i32), ("eps", ctypes.c_float), ("is_output_kv", _i32),
        ("k_rope", _p), ("c_kv", _p), ("k_rope_strides", _i64 * 3), ("c_kv_strides", _i64 * 3),
    ]


_lib.qknr_qk_norm_rope_across_heads.argtypes = [ctypes.POINTER(QkArgs), _p]
_lib.qknr_qk_norm_rope_across_heads.restype = _i32
_lib.qknr_qk_validate.argtypes = [ctypes.POINTER(QkArgs)]
_lib.qknr_qk_validate.restype = _i32
_lib.qknr_qk_sumsq_across_heads.argtypes = [ctypes.POINTER(QkArgs), _p, _p]
_lib.qknr_qk_sumsq_across_heads.restype = _i32
_lib.qknr_qk_apply_across_heads.argtypes = [ctypes.POINTER(QkArgs), _p, _p]
_lib.qknr_qk_apply_across_heads.restype = _i32
_lib.qknr_qk_norm_rope_per_head.argtypes = [ctypes.POINTER(QkArgs), _p]
_lib.qknr_qk_norm_rope_per_head.restype = _i32
_lib.qknr_interleaved_to_rotate_half.argtypes = [ctypes.POINTER(PermuteArgs), _p]
_lib.qknr_interleaved_to_rotate_half.restype = _i32
_lib.qknr_qkv_projection.argtypes = [ctypes.POINTER(ProjArgs), _p]
_lib.qknr_qkv_projection.restype = _i32
_lib.qknr_kv_rmsnorm_rope_cache.argtypes = [ctypes.POINTER(KvArgs), _p]
_lib.qknr_kv_rmsnorm_rope_cache.restype = _i32
_lib.qknr_kv_validate.argtypes = [ctypes.POINTER(KvArgs)]
_lib.qknr_kv_validate.restype = _i32
_lib.qknr_last_error.argtypes = []
_lib.qknr_last_error.restype = ctypes.c_char_p
_lib.qknr_version.argtypes = []
_lib.qknr_version.restype = _i32

EXPORTED = ("qknr_qk_norm_rope_across_heads", "qknr_qk_validate", "qknr_qk_sumsq_across_heads",
            "qknr_qk_apply_across_heads", "qknr_qk_norm_rope_per_head", "qknr_interleaved_to_rotate_half",
            "qknr_qkv_projection",
            "qknr_kv_rmsnorm_rope_cache", "qknr_kv_validate", "qknr_last_error", "qknr_version")


class QknrError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"qknr status {code}: {message}")
        self.code = code


def last_error() -> str:
    return _lib.qknr_last_error().decode()


def version() -> int:
    return int(_lib.qknr_version())


def _check(code: int):
    if code != OK:
        raise QknrError(code, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype(t) -> int:
    try:
        return _DTYPE[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _stream(device, stream):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _last_dim_contiguous(name, t):
    if t is not None and t.numel() > 0 and t.stride(-1) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")


# ----------------------------------------------------------------------------
# (a) across-heads QK RMSNorm + rotate-half RoPE
# ----------------------------------------------------------------------------

def qk_args(q, k, q_gamma, k_gamma, cos, sin, *, eps, q_out=None, k_out=None,
            apply_norm=True, apply_rope=True, per_head=False, q_norm_channels=0,
            k_norm_channels=0, sumsq_parts=0) -> QkArgs:
    """Fill ``qknr_qk_args`` from tensors.

    q: [B, S, n_q_heads, d] (any strides, d contiguous) -- e.g. a BSD projection
    ``qkv[..., :nq*d].unflatten(-1, (nq, d))`` or an NBSd buffer permuted to
    (B, S, N, d). k: [B, S, n_k_heads, d] with the same strides, or None.
    cos, sin: [B or 1, S, d] (a batch of 1 is shared). Outputs default to the
    inputs (in place). Gammas are [n_heads * d] (segment-wide) or, with
    ``per_head``, [d]. ``*_norm_channels``: the whole segment's channel count
    for the apply pass of a split norm (0 otherwise).
    """
    if q.dim() != 4:
        raise ValueError("q must be [B, S, n_q_heads, head_dim]")
    B, S, nq, d = q.shape
    q_out = q if q_out is None else q_out
    nk = 0
    if k is not None:
        if k.dim() != 4 or k.shape[0] != B or k.shape[1] != S or k.shape[3] != d:
            raise ValueError("k must be [B, S, n_k_heads, head_dim] like q")
        if k.stride() != q.stride():
            raise ValueError("q and k must share strides")
        nk = k.shape[2]
        k_out = k if k_out is None else k_out
        if k_out.stride() != q_out.stride():
            raise ValueError("q_out and k_out must share strides")
    if q_out.shape != q.shape:
        raise ValueError("q_out must have q's shape")
    for name, t in (("q", q), ("k", k), ("q_out", q_out), ("k_out", k_out), ("cos", cos), ("sin", sin)):
        _last_dim_contiguous(name, t)
    a = QkArgs()
    a.dtype = _dtype(q)
    for t in (k, q_out, k_out, q_gamma, k_gamma, cos, sin):
        if t is not None and t.dtype != q.dtype:
            raise TypeError("all tensors of (a) share one dtype")
    a.n_q_heads, a.n_k_heads, a.head_dim = nq, nk, d
    a.batch, a.seq = B, S
    a.q_in, a.k_in, a.q_out, a.k_out = _ptr(q), _ptr(k), _ptr(q_out), _ptr(k_out)
    a.in_batch_stride, a.in_token_stride, a.in_head_stride = q.stride(0), q.stride(1), q.stride(2)
    a.out_batch_stride, a.out_token_stride, a.out_head_stride = q_out.stride(0), q_out.stride(1), q_out.stride(2)
    if apply_norm:
        gq, gk = (d, d) if per_head else (nq * d, nk * d)
        if q_gamma is None or q_gamma.numel() != gq or (nk and (k_gamma is None or k_gamma.numel() != gk)):
            raise ValueError("gammas must be [head_dim] (per head)" if per_head else
                             "gammas must be [n_heads * head_dim] (segment-wide)")
        q_gamma = q_gamma.contiguous()
        k_gamma = k_gamma.contiguous() if nk else None
        a.q_gamma, a.k_gamma = _ptr(q_gamma), _ptr(k_gamma)
    if apply_rope:
        if (cos.dim() != 3 or cos.shape[0] not in (1, B) or cos.shape[1] != S or cos.shape[2] != d
                or sin.shape != cos.shape or cos.stride() != sin.stride()):
            raise ValueError("cos/sin must be [B or 1, S, head_dim] with equal strides")
        a.cos, a.sin = _ptr(cos), _ptr(sin)
        a.rope_batch_stride = 0 if cos.shape[0] == 1 else cos.stride(0)
        a.rope_token_stride = cos.stride(1)
    a.eps = float(eps)
    a.apply_norm, a.apply_rope = int(bool(apply_norm)), int(bool(apply_rope))
    a.q_norm_channels, a.k_norm_channels = int(q_norm_channels), int(k_norm_channels)
    a.sumsq_parts = int(sumsq_parts)
    a._keep = (q_gamma, k_gamma)  # keep contiguous copies alive
    return a


def qk_norm_rope_across_heads(q, k, q_gamma, k_gamma, cos, sin, *, eps, q_out=None, k_out=None,
                              apply_norm=True, apply_rope=True, stream=None):
    """Across-heads RMSNorm + rotate-half RoPE of Q and K (see :func:`qk_args`).
    Returns (q_out, k_out)."""
    if q_out is None:
        q_out = q
    if k is not None and k_out is None:
        k_out = k
    a = qk_args(q, k, q_gamma, k_gamma, cos, sin, eps=eps, q_out=q_out, k_out=k_out,
                apply_norm=apply_norm, apply_rope=apply_rope)
    with torch.cuda.device(q.device):
        _check(_lib.qknr_qk_norm_rope_across_heads(ctypes.byref(a), _stream(q.device, stream)))
    return q_out, k_out


def prepare_qk_norm_rope_across_heads(q, k, q_gamma, k_gamma, cos, sin, *, eps, q_out=None, k_out=None,
                                      apply_norm=True, apply_rope=True, stream=None):
    """Marshal the arguments once and return a zero-argument callable that
    launches (a) on the chosen stream (torch's current stream at preparation
    time by default). The tensors must stay alive and unmoved while the
    callable is used; each call re-validates on the host (a few microseconds)."""
    if q_out is None:
        q_out = q
    if k is not None and k_out is None:
        k_out = k
    a = qk_args(q, k, q_gamma, k_gamma, cos, sin, eps=eps, q_out=q_out, k_out=k_out,
                apply_norm=apply_norm, apply_rope=apply_rope)
    st = _stream(q.device, stream)
    ref = ctypes.byref(a)
    fn = _lib.qknr_qk_norm_rope_across_heads
    keep = (q, k, q_out, k_out, q_gamma, k_gamma, cos, sin)

    def launch():
        _check(fn(ref, st))
    launch.args, launch.tensors = a, keep
    return launch


def qk_validate(a: QkArgs) -> int:
    """Host-only validation of filled arguments; returns the status code."""
    return int(_lib.qknr_qk_validate(ctypes.byref(a)))


def qk_norm_rope_per_head(q, k, q_gamma, k_gamma, cos, sin, *, eps, q_out=None, k_out=None,
                          apply_norm=True, apply_rope=True, stream=None):
    """Per-head RMSNorm (gammas [head_dim] shared by every head) + rotate-half
    RoPE; arguments as :func:`qk_args`. Returns (q_out, k_out)."""
    if q_out is None:
        q_out = q
    if k is not None and k_out is None:
        k_out = k
    a = qk_args(q, k, q_gamma, k_gamma, cos, sin, eps=eps, q_out=q_out, k_out=k_out,
                apply_norm=apply_norm, apply_rope=apply_rope, per_head=True)
    with torch.cuda.device(q.device):
        _check(_lib.qknr_qk_norm_rope_per_head(ctypes.byref(a), _stream(q.device, stream)))
    return q_out, k_out


def qk_sumsq_across_heads(q, k=None, *, sumsq=None, stream=None):
    """Step a of a split across-heads norm: per token and segment, the sum of
    squares over the given heads. Returns fp32 [segs, B*S] (segs = 2 with k)."""
    B, S = q.shape[0], q.shape[1]
    segs = 2 if k is not None else 1
    if sumsq is None:
        sumsq = torch.empty(segs, B * S, dtype=torch.float32, device=q.device)
    if sumsq.dtype != torch.float32 or sumsq.numel() != segs * B * S or not sumsq.is_contiguous():
        raise ValueError(f"sumsq must be a contiguous float32 tensor of {segs}*B*S elements")
    a = qk_args(q, k, None, None, None, None, eps=0.0, apply_norm=False, apply_rope=False)
    a.q_out = a.k_out = None
    with torch.cuda.device(q.device):
        _check(_lib.qknr_qk_sumsq_across_heads(ctypes.byref(a), _ptr(sumsq), _stream(q.device, stream)))
    return sumsq


def _sum_parts(sumsq, q, segs):
    T = q.shape[0] * q.shape[1]
    if sumsq.dtype != torch.float32 or not sumsq.is_contiguous():
        raise ValueError("sumsq must be a contiguous float32 [segs, B*S, parts] (or [segs, B*S]) array")
    if T == 0:
        return 1
    if sumsq.numel() % (segs * T):
        raise ValueError("sumsq must hold segs * parts * B*S floats")
    return sumsq.numel() // (segs * T)


def qk_apply_across_heads(q, k, q_gamma, k_gamma, cos, sin, sumsq, *, eps, q_norm_channels,
                          k_norm_channels=0, q_out=None, k_out=None, apply_rope=True, stream=None):
    """Step c of a split across-heads norm on this rank's heads: ``sumsq``
    [segs, B*S] holds the sums added over every rank (or [segs, B*S, P]
    partial sums, added in a fixed order, e.g. the projection's per-tile sums),
    ``*_norm_channels`` the whole segment's channel count (n_heads*d*tp; 0:
    this call's own). Gammas are this rank's slice of the segment-wide gamma.
    Returns (q_out, k_out)."""
    if q_out is None:
        q_out = q
    if k is not None and k_out is None:
        k_out = k
    parts = _sum_parts(sumsq, q, 2 if k is not None else 1)
    a = qk_args(q, k, q_gamma, k_gamma, cos, sin, eps=eps, q_out=q_out, k_out=k_out, apply_norm=True,
                apply_rope=apply_rope, q_norm_channels=q_norm_channels, k_norm_channels=k_norm_channels,
                sumsq_parts=parts)
    with torch.cuda.device(q.device):
        _check(_lib.qknr_qk_apply_across_heads(ctypes.byref(a), _ptr(sumsq), _stream(q.device, stream)))
    return q_out, k_out


def _prepared(fn, a, extra, device, stream, keep):
    """A zero-argument launcher of `fn(&a, *extra, stream)` with the arguments
    marshalled once (the tensors in `keep` must stay alive and unmoved)."""
    st = _stream(device, stream)
    ref = ctypes.byref(a)

    def launch():
        _check(fn(ref, *extra, st))
    launch.args, launch.tensors = a, keep
    return launch


def prepare_qk_norm_rope_per_head(q, k, q_gamma, k_gamma, cos, sin, *, eps, q_out=None, k_out=None,
                                  apply_norm=True, apply_rope=True, stream=None):
    """Prepared form of :func:`qk_norm_rope_per_head`."""
    q_out = q if q_out is None else q_out
    k_out = k if (k is not None and k_out is None) else k_out
    a = qk_args(q, k, q_gamma, k_gamma, cos, sin, eps=eps, q_out=q_out, k_out=k_out,
                apply_norm=apply_norm, apply_rope=apply_rope, per_head=True)
    return _prepared(_lib.qknr_qk_norm_rope_per_head, a, (), q.device, stream,
                     (q, k, q_out, k_out, q_gamma, k_gamma, cos, sin))


def prepare_qk_sumsq_across_heads(q, k, sumsq, *, stream=None):
    """Prepared form of :func:`qk_sumsq_across_heads` writing into `sumsq`."""
    segs = 2 if k is not None else 1
    if sumsq.dtype != torch.float32 or sumsq.numel() != segs * q.shape[0] * q.shape[1] or not sumsq.is_contiguous():
        raise ValueError(f"sumsq must be a contiguous float32 tensor of {segs}*B*S elements")
    a = qk_args(q, k, None, None, None, None, eps=0.0, apply_norm=False, apply_rope=False)
    a.q_out = a.k_out = None
    return _prepared(_lib.qknr_qk_sumsq_across_heads, a, (_ptr(sumsq),), q.device, stream, (q, k, sumsq))


def prepare_qk_apply_across_heads(q, k, q_gamma, k_gamma, cos, sin, sumsq, *, eps, q_norm_channels,
                                  k_norm_channels=0, q_out=None, k_out=None, apply_rope=True, stream=None):
    """Prepared form of :func:`qk_apply_across_heads`."""
    q_out = q if q_out is None else q_out
    k_out = k if (k is not None and k_out is None) else k_out
    parts = _sum_parts(sumsq, q, 2 if k is not None else 1)
    a = qk_args(q, k, q_gamma, k_gamma, cos, sin, eps=eps, q_out=q_out, k_out=k_out, apply_norm=True,
                apply_rope=apply_rope, q_norm_channels=q_norm_channels, k_norm_channels=k_norm_channels,
                sumsq_parts=parts)
    return _prepared(_lib.qknr_qk_apply_across_heads, a, (_ptr(sumsq),), q.device, stream,
                     (q, k, q_out, k_out, q_gamma, k_gamma, cos, sin, sumsq))


def proj_args(a, w, bias, out, *, q_cols=0, k_cols=0, sumsq=None, a_scale=None, w_scale=None,
              a_block_scale=None, w_block_scale=None) -> ProjArgs:
    """Fill ``qknr_proj_args``: a [M, K], w [N, K] (a linear layer's weight),
    both bf16 or both float8_e4m3fn; bias [N] and out [M, N] bf16; a_scale [M]
    and w_scale [N] float32 or None; last dimensions contiguous. MXFP8:
    a_block_scale [M, K/32] and w_block_scale [N, K/32], E8M0 scale bytes
    (uint8 or float8_e8m0fnu), both given (scale_mode MX32) or both None."""
    if a.dim() != 2 or w.dim() != 2 or out.dim() != 2:
        raise ValueError("a, w and out must be 2-D ([M, K], [N, K], [M, N])")
    M, K = a.shape
    N = w.shape[0]
    if w.shape[1] != K or tuple(out.shape) != (M, N) or (bias is not None and bias.numel() != N):
        raise ValueError("shapes must be a [M, K], w [N, K], bias [N], out [M, N]")
    for name, t in (("a", a), ("w", w), ("out", out)):
        _last_dim_contiguous(name, t)
    if w.dtype != a.dtype or a.dtype not in (torch.bfloat16, torch.float8_e4m3fn):
        raise TypeError("a and w are both bfloat16 or both float8_e4m3fn")
    for t in (bias, out):
        if t is not None and t.dtype != torch.bfloat16:
            raise TypeError("bias and out are bfloat16")
    for name, t, n in (("a_scale", a_scale, M), ("w_scale", w_scale, N)):
        if t is not None and (t.dtype != torch.float32 or t.numel() != n or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 tensor of {n} elements")
    r = ProjArgs()
    r.dtype = _dtype(a)
    r.rows, r.in_features, r.out_features = M, K, N
    r.a, r.a_row_stride = _ptr(a), a.stride(0)
    r.w, r.w_row_stride = _ptr(w), w.stride(0)
    bias = bias.contiguous() if bias is not None else None
    r.bias = _ptr(bias)
    r.out, r.out_row_stride = _ptr(out), out.stride(0)
    r.q_cols, r.k_cols = q_cols, k_cols
    if q_cols:
        segs = 2 if k_cols else 1
        need = segs * (q_cols // 128) * M
        if sumsq is None or sumsq.dtype != torch.float32 or not sumsq.is_contiguous() or sumsq.numel() != need:
            raise ValueError(f"sumsq must be a contiguous float32 tensor of {need} elements")
    r.sumsq = _ptr(sumsq) if q_cols else None
    r.a_scale, r.w_scale = _ptr(a_scale), _ptr(w_scale)
    if (a_block_scale is None) != (w_block_scale is None):
        raise ValueError("a_block_scale and w_block_scale come together")
    if a_block_scale is not None:
        for name, t, n in (("a_block_scale", a_block_scale, M), ("w_block_scale", w_block_scale, N)):
            if t.dim() != 2 or t.shape[0] != n or t.shape[1] != K // 32 or t.element_size() != 1:
                raise ValueError(f"{name} must be a [{n}, {K // 32}] tensor of E8M0 bytes")
            _last_dim_contiguous(name, t)
        r.scale_mode = PROJ_SCALE_MX32
        r.a_block_scale, r.a_block_scale_stride = _ptr(a_block_scale), a_block_scale.stride(0)
        r.w_block_scale, r.w_block_scale_stride = _ptr(w_block_scale), w_block_scale.stride(0)
    else:
        r.scale_mode = PROJ_SCALE_ROW
    r._keep = (bias,)
    return r


def qkv_projection(a, w, bias=None, *, out=None, q_cols=0, k_cols=0, sumsq=None, a_scale=None, w_scale=None,
                   a_block_scale=None, w_block_scale=None, stream=None):
    """out = (a @ w.T) * a_scale[:, None] * w_scale[None, :] + bias on matrix
    cores (bf16 operands, or float8_e4m3fn operands with ROW_MX scales and/or
    MXFP8 block scales -- one E8M0 byte per 32 values of K on a and on w; the
    output is bf16), plus, for q_cols > 0, the
    per-row sums of squares of each 128-column tile of the Q columns
    [0, q_cols) and K columns [q_cols, q_cols + k_cols): fp32
    [segs, M, q_cols // 128], ready for :func:`qk_apply_across_heads`.
    Returns (out, sumsq)."""
    M, N = a.shape[0], w.shape[0]
    if out is None:
        out = torch.empty(M, N, dtype=torch.bfloat16, device=a.device)
    if q_cols and sumsq is None:
        sumsq = torch.empty(2 if k_cols else 1, M, q_cols // 128, dtype=torch.float32, device=a.device)
    r = proj_args(a, w, bias, out, q_cols=q_cols, k_cols=k_cols, sumsq=sumsq, a_scale=a_scale, w_scale=w_scale,
                  a_block_scale=a_block_scale, w_block_scale=w_block_scale)
    with torch.cuda.device(a.device):
        _check(_lib.qknr_qkv_projection(ctypes.byref(r), _stream(a.device, stream)))
    return out, sumsq


def prepare_qkv_projection(a, w, bias=None, *, out, q_cols=0, k_cols=0, sumsq=None, a_scale=None,
                           w_scale=None, a_block_scale=None, w_block_scale=None, stream=None):
    """Prepared form of :func:`qkv_projection` (arguments marshalled once)."""
    r = proj_args(a, w, bias, out, q_cols=q_cols, k_cols=k_cols, sumsq=sumsq, a_scale=a_scale, w_scale=w_scale,
                  a_block_scale=a_block_scale, w_block_scale=w_block_scale)
    return _prepared(_lib.qknr_qkv_projection, r, (), a.device, stream,
                     (a, w, bias, out, sumsq, a_scale, w_scale, a_block_scale, w_block_scale))


def permute_args(src, dst, head_dim, *, dim=-1, first=0, n_heads=None, inverse=False) -> PermuteArgs:
    """Fill ``qknr_permute_args`` for contiguous tensors src/dst of one shape."""
    if not (src.is_contiguous() and dst.is_contiguous()) or src.shape != dst.shape or src.dtype != dst.dtype:
        raise ValueError("src and dst must be contiguous tensors of one shape and dtype")
    dim = dim % src.dim()
    L = src.shape[dim]
    if n_heads is None:
        n_heads = (L - first) // head_dim
    outer = 1
    for n in src.shape[:dim]:
        outer *= n
    inner = 1
    for n in src.shape[dim + 1:]:
        inner *= n
    a = PermuteArgs()
    a.elem_bytes, a.inverse = src.element_size(), int(bool(inverse))
    a.outer, a.axis_len, a.inner = outer, L, inner
    a.first, a.n_heads, a.head_dim = first, n_heads, head_dim
    a.src, a.dst = _ptr(src), _ptr(dst)
    return a


def interleaved_to_rotate_half(src, head_dim, *, dim=-1, first=0, n_heads=None, inverse=False, out=None,
                               stream=None):
    """Permute `n_heads` blocks of `head_dim` indices of dimension `dim`,
    starting at `first`, from interleaved pairs (2j, 2j+1) to rotate-half
    pairs (j, j + d/2) (``inverse``: back); other indices are copied. For a
    fused QKV weight [H, I] use dim=1, n_heads = n_q + n_k; for interleaved
    cos/sin tables [.., d] the defaults. Returns the new tensor."""
    src = src.contiguous()
    if out is None:
        out = torch.empty_like(src)
    a = permute_args(src, out, head_dim, dim=dim, first=first, n_heads=n_heads, inverse=inverse)
    with torch.cuda.device(src.device):
        _check(_lib.qknr_interleaved_to_rotate_half(ctypes.byref(a), _stream(src.device, stream)))
    return out


# ----------------------------------------------------------------------------
# (b) KvRmsNormRopeCache
# ----------------------------------------------------------------------------

def _qshape(t, heads, width, v2):
    """Shape code of a quantisation parameter tensor: [1] -> SCALAR, [D] or
    [1, D] -> CHANNEL ([1, D] is [N, D] when V2 has N = 1), [N, D] -> HEAD_CHANNEL."""
    if t is None:
        return QSHAPE_SCALAR
    shape = tuple(t.shape)
    if shape == (1,):
        return QSHAPE_SCALAR
    if shape == (width,):
        return QSHAPE_CHANNEL
    if shape == (1, width):
        return QSHAPE_HEAD_CHANNEL if (v2 and heads == 1) else QSHAPE_CHANNEL
    if shape == (heads, width):
        return QSHAPE_HEAD_CHANNEL
    raise ValueError(f"quantisation parameter shape {shape} is not [1], [{width}], [1, {width}] "
                     f"or [{heads}, {width}]")


def _strides3(t):
    return (_i64 * 3)(*(t.stride()[:3] if t is not None else (0, 0, 0)))


def kv_args(kv, gamma, cos, sin, index, k_cache, ckv_cache, *, k_rope_scale=None, c_kv_scale=None,
            k_rope_offset=None, c_kv_offset=None, v=None, epsilon=1e-5, cache_mode="Norm",
            is_output_kv=False, k_rope=None, c_kv=None) -> KvArgs:
    """Fill ``qknr_kv_args`` from tensors named as on the KvRmsNormRopeCache
    parameter table.

    kv [Bkv, N, Skv, D]; v (v_optional) [Bkv, N, Skv, Dv] or None; gamma
    [rms_size]; cos/sin [Bkv, N, Skv or 1, rope]; index int64 ([Bkv, Skv] for
    Norm, [Bkv*Skv] for PA/PA_BNSD, [Bkv*ceil(Skv/block_size)] block starts for
    PA_BLK_BNSD); caches Norm [Bkv, N, Scache, D] or paged
    [block_num, block_size, N, D]; scales/offsets fp32 [1], [D], [1, D] (V1) or
    [N, D] (V2). V1 takes rope_size = cos.shape[-1] and rms_size = D - rope_size.
    """
    if kv.dim() != 4:
        raise ValueError("kv must be [Bkv, N, Skv, D]")
    B, N, S, D = kv.shape
    v2 = v is not None
    R = cos.shape[-1]
    a = KvArgs()
    a.dtype = _dtype(kv)
    for t in (gamma, cos, sin, v, k_rope, c_kv):
        if t is not None and t.dtype != kv.dtype:
            raise TypeError("kv, gamma, cos, sin, v_optional, k_rope and c_kv share one dtype")
    a.heads, a.batch, a.seq = N, B, S
    a.kv_dim, a.rope_size = D, R
    a.rms_size = D if v2 else D - R
    a.v_dim = v.shape[-1] if v2 else 0
    if cos.dim() != 4 or sin.shape != cos.shape or cos.stride() != sin.stride():
        raise ValueError("cos/sin must be 4-D with equal shapes and strides")
    for name, t in (("kv", kv), ("v_optional", v), ("cos", cos), ("sin", sin), ("k_cache", k_cache),
                    ("ckv_cache", ckv_cache), ("k_rope", k_rope), ("c_kv", c_kv)):
        _last_dim_contiguous(name, t)
    if gamma.numel() != a.rms_size:
        raise ValueError(f"gamma must have rms_size = {a.rms_size} elements")
    if index.dtype != torch.int64:
        raise TypeError("index must be int64")
    if cos.shape[0] != B or cos.shape[1] != N or cos.shape[2] not in (1, S):
        raise ValueError("cos/sin must be [Bkv, N, Skv or 1, rope_size]")
    if v2 and tuple(v.shape[:3]) != (B, N, S):
        raise ValueError("v_optional must be [Bkv, N, Skv, Dv]")
    dk_w = D if v2 else R
    dc_w = v.shape[-1] if v2 else D - R
    if cache_mode not in _CACHE_MODE:
        raise ValueError(f"cache_mode {cache_mode!r} is not built ({', '.join(_CACHE_MODE)})")
    if cache_mode == "Norm":
        if index.numel() != B * S or (index.dim() == 2 and tuple(index.shape) != (B, S)):
            raise ValueError("Norm index must be [Bkv, Skv]")
        lead_ok = (k_cache.dim() == 4 and ckv_cache.dim() == 4 and k_cache.shape[0] == B
                   and k_cache.shape[1] == N and tuple(ckv_cache.shape[:3]) == tuple(k_cache.shape[:3]))
    else:
        if k_cache.dim() != 4 or k_cache.shape[1] < 1:
            raise ValueError("paged caches must be [block_num, block_size, N, D]")
        entries = B * (-(-S // k_cache.shape[1]) if cache_mode == "PA_BLK_BNSD" else S)
        if index.numel() != entries:
            raise ValueError(f"{cache_mode} index must hold {entries} entries "
                             f"({'Bkv * ceil(Skv / block_size)' if cache_mode == 'PA_BLK_BNSD' else 'Bkv * Skv'})")
        lead_ok = (k_cache.dim() == 4 and ckv_cache.dim() == 4 and k_cache.shape[2] == N
                   and tuple(ckv_cache.shape[:3]) == tuple(k_cache.shape[:3]))
    if not lead_ok or k_cache.shape[3] != dk_w or ckv_cache.shape[3] != dc_w:
        raise ValueError(f"caches must be Norm [Bkv, N, Scache, D] or paged [block_num, block_size, N, D] "
                         f"with k width {dk_w} and ckv width {dc_w}, and agree in their leading dims")
    for name, t, w in (("k_rope", k_rope, dk_w), ("c_kv", c_kv, dc_w)):
        if t is not None and tuple(t.shape) != (B, N, S, w):
            raise ValueError(f"{name} must be [Bkv, N, Skv, {w}]")
    a.kv, a.v_optional = _ptr(kv), _ptr(v)
    gamma = gamma.contiguous()
    index = index.contiguous()
    a.gamma, a.cos, a.sin, a.index = _ptr(gamma), _ptr(cos), _ptr(sin), _ptr(index)
    a.kv_strides = _strides3(kv)
    a.v_strides = _strides3(v)
    rs = list(cos.stride()[:3])
    if cos.shape[2] == 1:
        rs[2] = 0  # S-axis broadcast (Srope = 1)
    a.rope_strides = (_i64 * 3)(*rs)
    a.cache_mode = _CACHE_MODE[cache_mode]
    a.k_cache, a.ckv_cache = _ptr(k_cache), _ptr(ckv_cache)
    a.k_cache_dtype, a.ckv_cache_dtype = _dtype(k_cache), _dtype(ckv_cache)
    if a.cache_mode == CACHE_NORM:
        # [Bkv, N, Scache, D] -> (batch, row, head)
        a.cache_rows = k_cache.shape[2]
        a.block_size = 0
        a.k_cache_strides = (_i64 * 3)(k_cache.stride(0), k_cache.stride(2), k_cache.stride(1))
        a.ckv_cache_strides = (_i64 * 3)(ckv_cache.stride(0), ckv_cache.stride(2), ckv_cache.stride(1))
    else:
        # [block_num, block_size, N, D] -> (block, slot in block, head)
        a.cache_rows = k_cache.shape[0]
        a.block_size = k_cache.shape[1]
        a.k_cache_strides = (_i64 * 3)(*k_cache.stride()[:3])
        a.ckv_cache_strides = (_i64 * 3)(*ckv_cache.stride()[:3])
    qp = [None if t is None else t.contiguous() for t in (k_rope_scale, k_rope_offset, c_kv_scale, c_kv_offset)]
    for t in qp:
        if t is not None and t.dtype != torch.float32:
            raise TypeError("quantisation parameters are float32")
    a.k_scale, a.k_offset, a.v_scale, a.v_offset = (_ptr(t) for t in qp)
    dk = D if v2 else R
    dc = a.v_dim if v2 else a.rms_size
    a.k_qshape, a.v_qshape = _qshape(qp[0], N, dk, v2), _qshape(qp[2], N, dc, v2)
    for scale, offset in ((qp[0], qp[1]), (qp[2], qp[3])):
        if scale is not None and offset is not None and scale.shape != offset.shape:
            raise ValueError("a scale and its offset must have the same shape")
    a.eps = float(epsilon)
    a.is_output_kv = int(bool(is_output_kv))
    a.k_rope, a.c_kv = _ptr(k_rope), _ptr(c_kv)
    a.k_rope_strides = _strides3(k_rope)
    a.c_kv_strides = _strides3(c_kv)
    a._keep = (gamma, index, qp)
    return a


def kv_rmsnorm_rope_cache(kv, gamma, cos, sin, index, k_cache, ckv_cache, *, k_rope_scale=None,
                          c_kv_scale=None, k_rope_offset=None, c_kv_offset=None, v=None,
                          epsilon=1e-5, cache_mode="Norm", is_output_kv=False, k_rope=None,
                          c_kv=None, stream=None):
    """KvRmsNormRopeCache: caches are updated in place; returns (k_rope, c_kv)
    when is_output_kv (allocating them if not given), else (None, None)."""
    if is_output_kv and (k_rope is None or c_kv is None):
        B, N, S, D = kv.shape
        R = cos.shape[-1]
        dk = D if v is not None else R
        dc = v.shape[-1] if v is not None else D - R
        if k_rope is None:
            k_rope = torch.empty((B, N, S, dk), dtype=kv.dtype, device=kv.device)
        if c_kv is None:
            c_kv = torch.empty((B, N, S, dc), dtype=kv.dtype, device=kv.device)
    a = kv_args(kv, gamma, cos, sin, index, k_cache, ckv_cache, k_rope_scale=k_rope_scale,
                c_kv_scale=c_kv_scale, k_rope_offset=k_rope_offset, c_kv_offset=c_kv_offset, v=v,
                epsilon=epsilon, cache_mode=cache_mode, is_output_kv=is_output_kv, k_rope=k_rope,
                c_kv=c_kv)
    with torch.cuda.device(kv.device):
        _check(_lib.qknr_kv_rmsnorm_rope_cache(ctypes.byref(a), _stream(kv.device, stream)))
    return (k_rope, c_kv) if is_output_kv else (None, None)


def prepare_kv_rmsnorm_rope_cache(kv, gamma, cos, sin, index, k_cache, ckv_cache, *, k_rope_scale=None,
                                  c_kv_scale=None, k_rope_offset=None, c_kv_offset=None, v=None,
                                  epsilon=1e-5, cache_mode="Norm", is_output_kv=False, k_rope=None,
                                  c_kv=None, stream=None):
    """Marshal the arguments of :func:`kv_rmsnorm_rope_cache` once and return a
    zero-argument callable that launches the operator (for decode loops and
    timing, where per-call Python marshalling would dominate a few-microsecond
    kernel). The tensors must stay alive and unmoved while it is used."""
    a = kv_args(kv, gamma, cos, sin, index, k_cache, ckv_cache, k_rope_scale=k_rope_scale,
                c_kv_scale=c_kv_scale, k_rope_offset=k_rope_offset, c_kv_offset=c_kv_offset, v=v,
                epsilon=epsilon, cache_mode=cache_mode, is_output_kv=is_output_kv, k_rope=k_rope,
                c_kv=c_kv)
    st = _stream(kv.device, stream)
    ref = ctypes.byref(a)
    fn = _lib.qknr_kv_rmsnorm_rope_cache
    keep = (kv, gamma, cos, sin, index, k_cache, ckv_cache, k_rope_scale, c_kv_scale, k_rope_offset,
            c_kv_offset, v, k_rope, c_kv)

    def launch():
        _check(fn(ref, st))
    launch.args, launch.tensors = a, keep
    return launch


def kv_validate(a: KvArgs) -> int:
    """Host-only validation of filled arguments; returns the status code."""
    return int(_lib.qknr_kv_validate(ctypes.byref(a)))
